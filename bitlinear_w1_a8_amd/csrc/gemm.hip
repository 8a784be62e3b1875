// Steps A2 + A3 for many tokens (prefill): a dense int8 contraction on the
// matrix cores.  Ternary weight tiles are expanded to int8 in LDS, as the
// 2B4T report (section 5.1) describes for its GPU kernel (packed in HBM,
// unpacked on chip, multiplied with 8-bit activations), and the result is
// rescaled in the epilogue.
//
// Tile: BM tokens x BN weight rows per block, K in steps of BK.  Per K step
// the block copies the int8 activation tile to LDS and expands the packed
// weight tile to signed int8 in LDS: (word >> 2j) & 0x03030303 isolates four
// codes c in {0,1,2}, and one byte-permute through the table {-1, 0, +1}
// turns them into t = c - 1.  Waves run v_mfma_i32_32x32x32_i8 with
// A = activations (rows = tokens) and B = weights (columns = output rows), so
// each lane's 16 results share one output column and a store of one register
// across the wave covers 32 consecutive outputs of a token.
#include "bl_internal.h"

namespace bl {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int kPad = 16;                 // bytes of padding per LDS row
constexpr int kLd = BK + kPad;
constexpr uint32_t kTernTable = 0x000100FFu;  // bytes {0xFF, 0x00, 0x01, 0x00}

__device__ __forceinline__ uint32_t signed_codes(uint32_t word, int j) {
  return __builtin_amdgcn_perm(kTernTable, kTernTable, codes_of(word, j));
}

__global__ __launch_bounds__(kThreads) void k_gemm(const uint32_t* __restrict__ packed,
                                                   const float* __restrict__ gamma,
                                                   const int8_t* __restrict__ xq,
                                                   const float* __restrict__ absmax, int T,
                                                   int N, int K, float* __restrict__ y,
                                                   int32_t* __restrict__ acc_out) {
  __shared__ __align__(16) int8_t As[BM * kLd];
  __shared__ __align__(16) int8_t Bs[BN * kLd];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ntn = (N + BN - 1) / BN;
  const int m0 = (blockIdx.x / ntn) * BM, n0 = (blockIdx.x % ntn) * BN;
  const int K16 = K >> 4;

  v16i acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;

  for (int k0 = 0; k0 < K; k0 += BK) {
    // activations: BM rows x BK bytes, 16 bytes per thread per step
#pragma unroll
    for (int u = 0; u < (BM * BK / 16) / kThreads; ++u) {
      const int id = tid + u * kThreads;
      const int row = id / (BK / 16), c16 = id % (BK / 16);
      const int tok = m0 + row, kk = k0 + c16 * 16;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (tok < T && kk < K) v = *reinterpret_cast<const uint4*>(xq + (int64_t)tok * K + kk);
      *reinterpret_cast<uint4*>(As + row * kLd + c16 * 16) = v;
    }
    // weights: BN rows x BK/16 packed words, expanded to 16 signed bytes each
#pragma unroll
    for (int u = 0; u < (BN * BK / 16) / kThreads; ++u) {
      const int id = tid + u * kThreads;
      const int row = id / (BK / 16), wj = id % (BK / 16);
      const int n = n0 + row, wi = (k0 >> 4) + wj;
      uint32_t w = 0;
      if (n < N && wi < K16) w = packed[(int64_t)n * K16 + wi];
      const uint4 e = make_uint4(signed_codes(w, 0), signed_codes(w, 1), signed_codes(w, 2),
                                 signed_codes(w, 3));
      *reinterpret_cast<uint4*>(Bs + row * kLd + wj * 16) = e;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int kb = ks * 32 + (lane >> 5) * 16;
      v4i a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint4 t = *reinterpret_cast<const uint4*>(As + (wm * 64 + i * 32 + (lane & 31)) * kLd + kb);
        a[i] = v4i{(int)t.x, (int)t.y, (int)t.z, (int)t.w};
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint4 t = *reinterpret_cast<const uint4*>(Bs + (wn * 64 + j * 32 + (lane & 31)) * kLd + kb);
        b[j] = v4i{(int)t.x, (int)t.y, (int)t.z, (int)t.w};
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  const float g = gamma[0];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int tok = m0 + wm * 64 + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
      if (tok >= T) continue;
      const float sc = out_scale(g, absmax[tok]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + wn * 64 + j * 32 + (lane & 31);
        if (n >= N) continue;
        const int64_t o = (int64_t)tok * N + n;
        const int s = acc[i][j][v];
        if (acc_out) acc_out[o] = s;
        y[o] = (float)s * sc;
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* packed, const float* gamma, const int8_t* xq,
                       const float* absmax, int64_t t, int64_t n, int64_t k, float* y,
                       int32_t* acc, hipStream_t stream) {
  const int64_t tiles = ((n + BN - 1) / BN) * ((t + BM - 1) / BM);
  const dim3 grid((unsigned)tiles);
  k_gemm<<<grid, kThreads, 0, stream>>>(reinterpret_cast<const uint32_t*>(packed), gamma, xq,
                                        absmax, (int)t, (int)n, (int)k, y, acc);
  return hipGetLastError();
}

}  // namespace bl
