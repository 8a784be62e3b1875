// Binary weights (+1 / -1, one bit each): step A0 and the decode kernel of
// steps A2 + A3.  The original BitNet has only these two weight values (the
// 2B4T explainer, section 2; "BitNet解读", on the zero weight); no page gives
// the rule, so the absmean scheme is kept with two levels: gamma = mean |W|,
// t = +1 where W >= 0 and -1 where W < 0, activations and rescale unchanged.
//
// Layout: weight k = 32g + 4j + i of a row sits at bit 8i + j of its
// little-endian word g (bit 1 = +1), so (w >> j) & 0x01010101 holds four
// consecutive k as bytes 0 / 1, an MFMA operand as it stands.  A row takes
// K / 8 bytes, half the ternary format.
//
// Contraction: the MFMA sums b * q with b in {0, 1}; since t = 2b - 1,
//   sum_k t q = 2 * sum_k b q - sum_k q,
// and the token sum of q over the same k is taken from the same activation
// bytes (one v_dot4 per 4 k), so the result is exact.
#include <algorithm>

#include "bl_internal.h"

namespace bl {
namespace {

// One thread per packed word: 32 weights, eight 16-byte loads.
__global__ __launch_bounds__(256) void k_binarize_pack(const float4* __restrict__ w,
                                                       int64_t nwords,
                                                       uint32_t* __restrict__ packed) {
  for (int64_t g = blockIdx.x * 256ll + threadIdx.x; g < nwords; g += (int64_t)gridDim.x * 256) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4 v = w[8 * g + j];   // k = 32g + 4j + i, i = 0..3
      word |= (uint32_t)(v.x >= 0.0f) << j;
      word |= (uint32_t)(v.y >= 0.0f) << (8 + j);
      word |= (uint32_t)(v.z >= 0.0f) << (16 + j);
      word |= (uint32_t)(v.w >= 0.0f) << (24 + j);
    }
    packed[g] = word;
  }
}

// Decode kernel for T <= 16, int8 activations, K % 256 == 0.  The structure is
// that of the ternary decode kernel on int8 input: a block owns 16 rows, wave
// w a contiguous run of at most CPW chunks (16 packed words = 512 k of each
// row, the last one possibly half), the activations of its run go global ->
// LDS first and every weight load of the run is issued at once; partial 16 x
// 16 tiles meet through LDS atomics and the last wave writes the outputs.
//
// v_mfma_i32_16x16x64_i8: lane (qg, r) feeds row r and token column r with
// the 128 k of words 4qg .. 4qg + 3 of the chunk; slice j of those words
// (bits j of each byte) pairs with dword 8v + j of the lane's 128 activation
// bytes.  The words are shifted down by 2p (p = 0..3) and masked in place:
// mask 0x01 gives slice 2p as b, mask 0x02 slice 2p + 1 as 2b, into two
// accumulators; the second one's exact sum is halved at the end.
constexpr int kBinChunk = 512;                          // k per chunk
constexpr int kBinHead = 32 * 4 + 256 * 4 + 4 + 12;     // zeros, tile, counter (16-byte padded)
static_assert(kBinHead % 16 == 0, "LDS header alignment");

typedef __attribute__((address_space(3))) void* bin_lds_t;
typedef __attribute__((address_space(1))) void* bin_glb_t;

template <int CPW>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(CPW == 8 ? 6 : 8))) void k_gemv_bin(
    const uint32_t* __restrict__ packed, const float* __restrict__ gamma,
    const int8_t* __restrict__ xq, const float* __restrict__ absmax, int T, int N, int K,
    int per, float* __restrict__ y, int32_t* __restrict__ acc_out) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int nwaves = blockDim.x >> 6;
  const int n0 = (int)blockIdx.x * 16;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qg = lane >> 4, r = lane & 15;
  const int K32 = K >> 5;                           // packed words per row
  const int nchunks = (K + kBinChunk - 1) / kBinChunk;
  const int c0 = wave * per;
  const int cnt = min(per, nchunks - c0);           // <= 0 when K is narrower than the block

  int* zero = reinterpret_cast<int*>(smem);         // 32 ints of zeros
  int* tile = zero + 32;                            // [token][row]
  int* counter = tile + 256;
  const int tstride = K + 16;
  unsigned char* xs8 = smem + kBinHead;             // [T][K + 16] int8 activations

  const int n = n0 + r < N ? n0 + r : N - 1;        // rows past N are computed, never stored
  const uint32_t* wrow = packed + (int64_t)n * K32;

  // this wave's activation run (all tokens), straight into LDS
  const int run0 = c0 * kBinChunk;
  const int runb = cnt > 0 ? min(cnt * kBinChunk, K - run0) : 0;
  for (int t = 0; t < T; ++t)
    for (int base = 0; base < runb; base += 1024)
      if (base + 16 * lane < runb)
        __builtin_amdgcn_global_load_lds((bin_glb_t)(xq + (int64_t)t * K + run0 + base + 16 * lane),
                                         (bin_lds_t)(xs8 + t * tstride + run0 + base), 16, 0, 0);
  const float g = gamma[0];
  // then every weight chunk of the run; a lane whose words lie past the row
  // (the upper half of a half chunk) or a slot past cnt reads word 0 and meets
  // a zero B operand
  uint4 buf[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    int wi = 16 * (c0 + i) + 4 * qg;
    wi = (i < cnt && wi + 4 <= K32) ? wi : 0;
    buf[i] = *reinterpret_cast<const uint4*>(wrow + wi);
  }
  for (int i = threadIdx.x; i < 32 + 256 + 1; i += nwaves * 64) zero[i] = 0;
  lds_sync();                                       // header cleared
  wait_vmem<CPW>();                                 // this wave's activation run landed

  int qsum = 0;   // sum of q over this wave's run, token of lane l: l & 15
  for (int t = 0; t < T; ++t) {
    const uint4* xt = reinterpret_cast<const uint4*>(xs8 + t * tstride + run0);
    int part = 0;
    for (int i = lane; i < runb / 16; i += 64) {
      const uint4 v = xt[i];
      part = __builtin_amdgcn_sdot4((int)v.x, 0x01010101, part, false);
      part = __builtin_amdgcn_sdot4((int)v.y, 0x01010101, part, false);
      part = __builtin_amdgcn_sdot4((int)v.z, 0x01010101, part, false);
      part = __builtin_amdgcn_sdot4((int)v.w, 0x01010101, part, false);
    }
    const int sum = wave_sum_i(part);
    if (r == t) qsum = sum;
  }

  const unsigned char* xrow = xs8 + (r < T ? r : 0) * tstride + qg * 128;
  v4i acc1 = {0, 0, 0, 0}, acc2 = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int c = c0 + i;
    const bool ok = r < T && i < cnt && 16 * c + 4 * qg + 4 <= K32;
    const uint32_t* xc = ok ? reinterpret_cast<const uint32_t*>(xrow + c * kBinChunk)
                            : reinterpret_cast<const uint32_t*>(zero);
    auto xs = [&](int j) { return v4i{(int)xc[j], (int)xc[8 + j], (int)xc[16 + j], (int)xc[24 + j]}; };
    const uint4 w4 = buf[i];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint4 ws = make_uint4(w4.x >> (2 * p), w4.y >> (2 * p), w4.z >> (2 * p), w4.w >> (2 * p));
      acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(
          (v4i{(int)(ws.x & 0x01010101u), (int)(ws.y & 0x01010101u), (int)(ws.z & 0x01010101u),
               (int)(ws.w & 0x01010101u)}),
          xs(2 * p), acc1, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(
          (v4i{(int)(ws.x & 0x02020202u), (int)(ws.y & 0x02020202u), (int)(ws.z & 0x02020202u),
               (int)(ws.w & 0x02020202u)}),
          xs(2 * p + 1), acc2, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);   // one chunk's operands live at a time
  }

  // lane (qg, r) holds rows 4qg + v of token column r: sum t q = 2 sum b q - sum q
  if (r < T) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int sb = acc1[v] + (acc2[v] >> 1);
      atomicAdd(&tile[r * 16 + 4 * qg + v], 2 * sb - qsum);
    }
  }
  int ticket = 0;
  if (lane == 0)
    ticket = __hip_atomic_fetch_add(counter, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
  ticket = __builtin_amdgcn_readfirstlane(ticket);
  if (ticket != nwaves - 1) return;
  for (int idx = lane; idx < 16 * T; idx += 64) {
    const int i = idx & 15, tl = idx >> 4;
    const int nn = n0 + i;
    if (nn >= N) continue;
    const int sum = __hip_atomic_load(&tile[idx], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const int64_t o = (int64_t)tl * N + nn;
    if (acc_out) acc_out[o] = sum;
    y[o] = (float)sum * out_scale(g, absmax[tl]);
  }
}

int grid_for(int64_t items, int threads, int cap) {
  int64_t g = (items + threads - 1) / threads;
  return (int)std::max<int64_t>(1, std::min<int64_t>(g, cap));
}

// Shapes the binary decode kernel takes (int8 activations of T tokens staged in LDS).
bool bin_dec_ok(int64_t t, int64_t k) { return t <= 16 && t * k <= 32768 && k % 256 == 0; }

hipError_t run_gemv_bin(const uint8_t* packed, const float* gamma, const int8_t* xq,
                        const float* absmax, int t, int n, int k, float* y, int32_t* acc,
                        hipStream_t stream) {
  const int blocks = (n + 15) / 16;
  const int nchunks = (k + kBinChunk - 1) / kBinChunk;
  // about two chunks per wave, at most 8 waves per block and no more waves
  // than fit at once (8 per SIMD), never more than 8 chunks per wave
  int nw = std::min((nchunks + 1) / 2, 8);
  const int fit = 8192 / blocks;
  if (nw > fit) nw = fit > 1 ? fit : 1;
  nw = std::max(nw, (nchunks + 7) / 8);
  const int per = (nchunks + nw - 1) / nw;
  const size_t lds = kBinHead + (size_t)t * (k + 16);
  const uint32_t* pw = reinterpret_cast<const uint32_t*>(packed);
  if (per <= 2)
    k_gemv_bin<2><<<blocks, nw * 64, lds, stream>>>(pw, gamma, xq, absmax, t, n, k, per, y, acc);
  else if (per <= 4)
    k_gemv_bin<4><<<blocks, nw * 64, lds, stream>>>(pw, gamma, xq, absmax, t, n, k, per, y, acc);
  else
    k_gemv_bin<8><<<blocks, nw * 64, lds, stream>>>(pw, gamma, xq, absmax, t, n, k, per, y, acc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_binary(const float* w, int64_t n, int64_t k, uint8_t* packed,
                              float* gamma, unsigned long long* buckets, hipStream_t stream) {
  hipError_t e = launch_gamma(w, n, k, gamma, buckets, stream);
  if (e != hipSuccess) return e;
  const int64_t nwords = n * k / 32;
  k_binarize_pack<<<grid_for(nwords, 256, 65536), 256, 0, stream>>>(
      reinterpret_cast<const float4*>(w), nwords, reinterpret_cast<uint32_t*>(packed));
  return hipGetLastError();
}

hipError_t launch_forward_binary(const uint8_t* packed, const float* gamma, const int8_t* xq,
                                 const float* absmax, int64_t t, int64_t n, int64_t k, float* y,
                                 int32_t* acc, int algo, hipStream_t stream) {
  // BL_ALGO_GEMV: the decode kernel, 16 tokens (or as many as fit LDS) per launch
  if (algo == BL_ALGO_GEMV || (algo == BL_ALGO_AUTO && bin_dec_ok(t, k))) {
    const int64_t tg = std::max<int64_t>(1, std::min<int64_t>(16, 32768 / k));
    for (int64_t t0 = 0; t0 < t; t0 += tg) {
      const int tc = (int)std::min(tg, t - t0);
      hipError_t e = run_gemv_bin(packed, gamma, xq + t0 * k, absmax + t0, tc, (int)n, (int)k,
                                  y + t0 * n, acc ? acc + t0 * n : nullptr, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  return launch_gemm_binary(packed, gamma, xq, absmax, t, n, k, y, acc, stream);
}

}  // namespace bl
