// Internal declarations shared by the HIP translation units of libbitlinear.
// Nothing here is part of the public C ABI (include/bitlinear.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bitlinear.h"

namespace bl {

// Constants of the forward.  eps is added to gamma before the weight division
// and floors a token's absmax; activations are clipped to [-127, 127].
constexpr float kEps = 1e-5f;
constexpr float kQb = 127.0f;

// Largest T that the automatic choice sends to the decode kernel (auto_algo:
// 64 for matrices of up to 2 MB packed, 32 up to 16 MB, 6 beyond).
constexpr int64_t kGemvMaxTokens = 64;

// Compute units of the current device (looked up once per device).
int device_cus();

// The automatic kernel choice of bitlinear_forward: BL_ALGO_GEMV (the decode
// kernels) or BL_ALGO_GEMM (the tiled MFMA kernel), by shape (gemv.hip).
int auto_algo(int64_t t, int64_t n, int64_t k);

// Measurement helpers (calib.hip): the launch floor, the HBM read stream and
// the int8 matrix-core rate of the device; the read writes one sink entry per
// wave (kCalibReadBlocks blocks of four), the MFMA loop kCalibMfmaWaves.
constexpr int kCalibReadBlocks = 1024;
constexpr int kCalibMfmaWaves = 4096;
constexpr int64_t kCalibSinkLen = 4096;
hipError_t launch_calib_empty(hipStream_t stream);
constexpr int kReadChunks = 0, kReadStride = 1;   // bl_read_layout
hipError_t launch_calib_read(const void* buf, int64_t bytes, int layout, uint32_t* sink,
                             hipStream_t stream);
hipError_t launch_calib_mfma(int iters, int byte, int32_t* sink, hipStream_t stream);

// Exponent buckets of the exact gamma sum: one uint64 per binary32 exponent.
constexpr int kGammaBuckets = 256;
constexpr size_t kPackWorkspaceBytes = kGammaBuckets * sizeof(unsigned long long);

hipError_t launch_pack(const float* w, int64_t n, int64_t k, uint8_t* packed, float* gamma,
                       unsigned long long* buckets, hipStream_t stream);

// Device address of the library's own kGammaBuckets buckets on the device of
// `stream` (the current device for the null stream), looked up once per device.
hipError_t scratch_buckets(hipStream_t stream, unsigned long long** out);

// gamma = mean |W| alone (exact sum, one rounding), shared by both weight formats.
hipError_t launch_gamma(const float* w, int64_t n, int64_t k, float* gamma,
                        unsigned long long* buckets, hipStream_t stream);

// Binary weights (+1 / -1, one bit each): step A0, and steps A2 + A3 (K % 256 == 0).
hipError_t launch_pack_binary(const float* w, int64_t n, int64_t k, uint8_t* packed,
                              float* gamma, unsigned long long* buckets, hipStream_t stream);
hipError_t launch_forward_binary(const uint8_t* packed, const float* gamma, const int8_t* xq,
                                 const float* absmax, int64_t t, int64_t n, int64_t k, float* y,
                                 int32_t* acc, int algo, hipStream_t stream);
// The tiled MFMA kernel on one-bit weights (any T, K % 128 == 0).
hipError_t launch_gemm_binary(const uint8_t* packed, const float* gamma, const int8_t* xq,
                              const float* absmax, int64_t t, int64_t n, int64_t k, float* y,
                              int32_t* acc, hipStream_t stream);

hipError_t launch_quant(const void* x, int bf16, int64_t t, int64_t k, int8_t* xq,
                        float* absmax, int32_t* rowsum, hipStream_t stream);

// Sub-layer norm (RMS with gain) in front of step A1; scale[t] gets the
// token's dequantisation absmax r * max|x * g|.
hipError_t launch_subln_quant(const void* x, int bf16, const float* gain, float eps_n, int64_t t,
                              int64_t k, int8_t* xq, float* scale, int32_t* rowsum,
                              hipStream_t stream);

// Decode kernel: handles any T by taking tokens 64 at a time.  rowsum (the
// tokens' sums of q) may be NULL: the kernel then derives the sums itself.
hipError_t launch_gemv(const uint8_t* packed, const float* gamma, const int8_t* xq,
                       const float* absmax, const int32_t* rowsum, int64_t t, int64_t n,
                       int64_t k, float* y, int32_t* acc, hipStream_t stream);

// Table-lookup decode kernel (comparison design), any T (one token per block row).
hipError_t launch_gemv_lut(const uint8_t* packed, const float* gamma, const int8_t* xq,
                           const float* absmax, int64_t t, int64_t n, int64_t k, float* y,
                           int32_t* acc, hipStream_t stream);

// Packed-int8-dot decode kernel (comparison design), any T (one token per block row).
hipError_t launch_gemv_dot4(const uint8_t* packed, const float* gamma, const int8_t* xq,
                            const float* absmax, int64_t t, int64_t n, int64_t k, float* y,
                            int32_t* acc, hipStream_t stream);

// Steps A1-A3 for a group of problems (bitlinear_linear_grouped).
hipError_t launch_linear_group(const struct bl_linear* probs, int count, int64_t t, int bf16,
                               hipStream_t stream);

// Tiled MFMA kernel, any T; rowsum as for launch_gemv.
hipError_t launch_gemm(const uint8_t* packed, const float* gamma, const int8_t* xq,
                       const float* absmax, const int32_t* rowsum, int64_t t, int64_t n,
                       int64_t k, float* y, int32_t* acc, hipStream_t stream);

// Gate and up projections of one input with the gated ReLU^2 epilogue: the
// packed matrix holds 2n rows, row 2i of the gate and row 2i+1 of the up
// projection; h is [t, n / 2] bfloat16; acc, when given, the [t, n] exact sums.
hipError_t launch_gated(const void* x, int bf16, const uint8_t* packed, const float* gamma_gate,
                        const float* gamma_up, int64_t t, int64_t n, int64_t k, uint16_t* h,
                        int8_t* xq, float* absmax, int32_t* acc, hipStream_t stream);

// The int8-input kernels of the gated path: the decode kernels (t <= 64) and
// the tiled MFMA kernel.
hipError_t launch_gemv_gated(const uint8_t* packed, const float* gamma_gate,
                             const float* gamma_up, const int8_t* xq, const float* absmax,
                             int64_t t, int64_t n, int64_t k, uint16_t* h, int32_t* acc,
                             hipStream_t stream);
hipError_t launch_gemm_gated(const uint8_t* packed, const float* gamma_gate,
                             const float* gamma_up, const int8_t* xq, const float* absmax,
                             int64_t t, int64_t n, int64_t k, uint16_t* h, int32_t* acc,
                             hipStream_t stream);

// Rows of two packed matrices interleaved: out row 2i = a row i, 2i+1 = b row i.
hipError_t launch_interleave(const uint8_t* a, const uint8_t* b, int64_t n, int64_t k,
                             uint8_t* out, hipStream_t stream);

// ---------------------------------------------------------------- device helpers

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// Codes of weights k = 16g+4j .. 16g+4j+3 of a packed word, one per byte.
__device__ __forceinline__ uint32_t codes_of(uint32_t word, int j) {
  return (word >> (2 * j)) & 0x03030303u;
}

// Binary32 scale applied to a token's exact int32 sum: gamma * m / 127.
__device__ __forceinline__ float out_scale(float gamma, float absmax) {
  const float m = fmaxf(absmax, kEps);
  return (gamma * m) / kQb;
}

// DPP row reductions (16 lanes), then the four rows through readlane.
__device__ __forceinline__ int wave_max_nonneg(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false));  // row_mirror
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ uint32_t wave_xor_u(uint32_t u) {
  int v = (int)u;
  v ^= __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  v ^= __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  v ^= __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
  v ^= __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);
  return (uint32_t)(__builtin_amdgcn_readlane(v, 0) ^ __builtin_amdgcn_readlane(v, 16) ^
                    __builtin_amdgcn_readlane(v, 32) ^ __builtin_amdgcn_readlane(v, 48));
}
__device__ __forceinline__ int wave_sum_i(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
         __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

// Block barrier for LDS traffic only.  __syncthreads() also orders global
// memory, and on this target loads and stores share one counter, so it would
// wait for every weight load in flight.  The empty asm statements keep the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_sync() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt not waited on
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));   // lgkmcnt, expcnt: no wait
}

// Exact non-negative integers in L little-endian 32-bit limbs (the exact
// sums of gamma and of the SubLN squares), used by one thread.
//
// limbs_add: add v * 2^off (off >= 0); the caller guarantees that the sum fits.
template <int L>
__device__ __forceinline__ void limbs_add(uint32_t (&limb)[L], unsigned long long v, int off) {
  if (!v) return;
  const int l0 = off >> 5, o = off & 31;
  const unsigned long long lo = v << o;
  const uint32_t part[3] = {(uint32_t)lo, (uint32_t)(lo >> 32), o ? (uint32_t)(v >> (64 - o)) : 0u};
  unsigned long long carry = 0;
  for (int i = l0; i < L; ++i) {
    const int pi = i - l0;
    const unsigned long long s = (unsigned long long)limb[i] + carry + (pi < 3 ? part[pi] : 0u);
    limb[i] = (uint32_t)s;
    carry = s >> 32;
    if (pi >= 2 && !carry) break;
  }
}

// limbs_to_f64: the integer times 2^scale, rounded once to binary64 (nearest,
// ties to even); the result must lie in the normal binary64 range or be 0.
// Word-wise: the top four limbs give the significand, the round bit and part
// of the sticky bit, the limbs below only the rest of the sticky bit.  (A
// bit-by-bit scan for the sticky bit ran through hundreds of zero bits of a
// sum of bf16 squares, in scratch memory, and cost tens of microseconds.)
template <int L>
__device__ __forceinline__ double limbs_to_f64(const uint32_t (&limb)[L], int scale) {
  int tw = -1;
  for (int i = L - 1; i >= 0; --i)
    if (limb[i]) { tw = i; break; }
  if (tw < 0) return 0.0;
  const int top = tw * 32 + (31 - __builtin_clz(limb[tw]));
  if (top <= 52) {
    const unsigned long long x = ((unsigned long long)limb[1] << 32) | limb[0];
    return ldexp((double)x, scale);
  }
  // the 128-bit window of limbs tw .. tw - 3 (missing ones are 0), bit 0 at
  // bit 32 (tw - 3) of the integer, shifted so that its top bit is bit 127
  unsigned long long hi = ((unsigned long long)limb[tw] << 32) | (tw >= 1 ? limb[tw - 1] : 0u);
  unsigned long long lo = ((unsigned long long)(tw >= 2 ? limb[tw - 2] : 0u) << 32) |
                          (tw >= 3 ? limb[tw - 3] : 0u);
  bool sticky = false;
  for (int i = tw - 4; i >= 0; --i) sticky |= limb[i] != 0u;
  const int lz = __builtin_clzll(hi);
  if (lz) {
    hi = (hi << lz) | (lo >> (64 - lz));
    lo <<= lz;
  }
  unsigned long long m = hi >> 11;                  // 53 bits
  const unsigned long long rem = hi & 0x7ffull;
  const bool rnd = (rem >> 10) & 1ull;
  sticky |= (rem & 0x3ffull) != 0 || lo != 0;
  int e = (tw - 3) * 32 - lz + 75;                  // weight of m's lowest bit
  if (rnd && (sticky || (m & 1ull))) {
    ++m;
    if (m == (1ull << 53)) { m >>= 1; ++e; }
  }
  return ldexp((double)m, e + scale);
}

// (s2:s1:s0) * 2^scale rounded once to binary64 (nearest, ties to even), in
// registers; the result must lie in the normal binary64 range or be 0.
__device__ __forceinline__ double u192_to_f64(unsigned long long s0, unsigned long long s1,
                                              unsigned long long s2, int scale) {
  unsigned long long hi, lo;
  bool sticky = false;
  int base;                                         // bit of the integer at lo's bit 0
  if (s2) { hi = s2; lo = s1; sticky = s0 != 0; base = 64; }
  else if (s1) { hi = s1; lo = s0; base = 0; }
  else {
    if (s0 < (1ull << 53)) return ldexp((double)s0, scale);
    hi = s0; lo = 0; base = -64;
  }
  const int lz = __builtin_clzll(hi);
  if (lz) {
    hi = (hi << lz) | (lo >> (64 - lz));
    lo <<= lz;
  }
  unsigned long long m = hi >> 11;                  // 53 bits
  const unsigned long long rem = hi & 0x7ffull;
  const bool rnd = (rem >> 10) & 1ull;
  sticky |= (rem & 0x3ffull) != 0 || lo != 0;
  int e = base - lz + 75;                           // weight of m's lowest bit
  if (rnd && (sticky || (m & 1ull))) {
    ++m;
    if (m == (1ull << 53)) { m >>= 1; ++e; }
  }
  return ldexp((double)m, e + scale);
}

// gamma * max(absmax, eps), exact in binary64 (two 24-bit significands).
__device__ __forceinline__ double gamma_m(float gamma, float absmax) {
  return (double)gamma * (double)fmaxf(absmax, kEps);
}

// Step A3 in binary64, rounded to binary32: RN32(RN64(RN64(acc * gamma * m) / 127)),
// the oracle's rescale of the sum, with gm = gamma * m from gamma_m.  acc * gm
// is one rounding of the exact product (acc * gamma is exact in binary64).
// The division by 127 is a product with RN64(1/127), then a correction by
// the exact remainder (one fused multiply-add), which is correctly rounded
// here: t / 127 of a 53-bit t is never a binary64 midpoint and lies at least
// ulp/254 from one, far more than the error of the corrected quotient.
__device__ __forceinline__ float a3_f32(int acc, double gm) {
  constexpr double kInv = 1.0 / 127.0;          // RN64(1/127)
  const double t = (double)acc * gm;
  const double q0 = t * kInv;
  const double rem = fma(-q0, 127.0, t);        // exact: q0 is within one ulp of t / 127
  return (float)fma(rem, kInv, q0);
}

// Gated ReLU^2 of one output pair, rounded to bfloat16 (nearest, ties to
// even): g and u are the binary32 roundings of step A3's binary64 value
// (a3_f32, gm_g and gm_u from gamma_m), h = (max(g, 0)^2) * u with the two
// binary32 products in that order.
__device__ __forceinline__ uint16_t gated_relu2_bf16(int acc_g, int acc_u, double gm_g,
                                                     double gm_u) {
  const float g = a3_f32(acc_g, gm_g), u = a3_f32(acc_u, gm_u);
  const float r = fmaxf(g, 0.0f);
  const float h = (r * r) * u;
  uint32_t b = __float_as_uint(h);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

}  // namespace bl
