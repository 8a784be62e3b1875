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

// T at or below which the automatic choice takes the decode kernel: measured
// on 2560->6912 and 6912->2560 against the tiled MFMA kernel with its tile
// choice, the decode kernel is faster through T = 32 on both, within 5% at
// T = 64 (faster on one, slower on the other) and twice as slow at T = 128.
constexpr int64_t kGemvMaxTokens = 64;

// Measurement helpers (calib.hip): the launch floor, the HBM read stream and
// the int8 matrix-core rate of the device; the read writes kCalibReadBlocks
// sink entries, the MFMA loop kCalibMfmaWaves.
constexpr int kCalibReadBlocks = 2048;
constexpr int kCalibMfmaWaves = 4096;
constexpr int64_t kCalibSinkLen = 4096;
hipError_t launch_calib_empty(hipStream_t stream);
hipError_t launch_calib_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream);
hipError_t launch_calib_mfma(int iters, int byte, int32_t* sink, hipStream_t stream);

// Exponent buckets of the exact gamma sum: one uint64 per binary32 exponent.
constexpr int kGammaBuckets = 256;
constexpr size_t kPackWorkspaceBytes = kGammaBuckets * sizeof(unsigned long long);

hipError_t launch_pack(const float* w, int64_t n, int64_t k, uint8_t* packed, float* gamma,
                       unsigned long long* buckets, hipStream_t stream);

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

// Decode kernel: handles any T by taking tokens 64 at a time.
hipError_t launch_gemv(const uint8_t* packed, const float* gamma, const int8_t* xq,
                       const float* absmax, int64_t t, int64_t n, int64_t k, float* y,
                       int32_t* acc, hipStream_t stream);

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

hipError_t launch_gemm(const uint8_t* packed, const float* gamma, const int8_t* xq,
                       const float* absmax, int64_t t, int64_t n, int64_t k, float* y,
                       int32_t* acc, hipStream_t stream);

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

// Gated ReLU^2 of one output pair, rounded to bfloat16 (nearest, ties to
// even): g = acc_g * sg and u = acc_u * su (binary32), h = (max(g, 0)^2) * u
// with the two products in that order.
__device__ __forceinline__ uint16_t gated_relu2_bf16(int acc_g, int acc_u, float sg, float su) {
  const float g = (float)acc_g * sg, u = (float)acc_u * su;
  const float r = fmaxf(g, 0.0f);
  const float h = (r * r) * u;
  uint32_t b = __float_as_uint(h);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

}  // namespace bl
