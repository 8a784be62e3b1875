// Steps A2 + A3 by table lookup: a decode kernel built the way the CPU
// lookup-table kernels of bitnet.cpp work (TL1 / TL2 in "微软 BitNet 在 x86/ARM
// CPU 上实现 2–6 倍推理加速", section 1.3: products replaced by table lookups),
// kept as a comparison point for the matrix-core decode kernel.
//
// Two weights of a row that share a 4-bit nibble of the packed layout (k and
// k + 4: byte i of word g holds k = 16g + i + 4j at bits 2j, so nibble h pairs
// j = 2h and 2h + 1) take one of nine code pairs.  Per token and per such
// pair of activation positions the block tabulates all sixteen nibble values
//   tab[nibble] = (ca - 1) * x[ka] + (cb - 1) * x[kb]   (0 for the unused code 3),
// and each weight row then needs one LDS lookup and one add per two weights,
// with no multiply and no unpacking beyond extracting the nibble.  The sums
// are exact int32, so the outputs equal the other kernels' bit for bit.
//
// Layout: a block owns 16 rows and its four waves split K; four lanes share a
// row and read 64 contiguous bytes of it per load (16 rows x 64 bytes per wave
// instruction).  K is taken 2048 at a time: the table of one chunk is 128
// packed words x 8 nibble positions x 16 entries of int16, 33 KB with a
// 4-entry pad per word so that the four lanes of a row (words 4 apart) hit
// different LDS banks; all four waves build it, each wave then looks up its
// quarter of the chunk, and the four partial sums of a row meet in LDS.
#include "bl_internal.h"

namespace bl {
namespace {

constexpr int kLutK = 2048;                  // k per table chunk
constexpr int kLutWords = kLutK / 16;        // packed words per row per chunk
constexpr int kLutWordStride = 8 * 16 + 4;   // int16 entries per word, padded
constexpr int kLutWaves = 4;
constexpr int kLutThreads = kLutWaves * 64;
constexpr int kLutVecs = kLutWords / 4 / 4 / kLutWaves;   // 16-byte vectors per lane per chunk
constexpr int kLutGroups = kLutWords * 8 / kLutThreads;   // table groups per thread

template <bool VEC4>
__global__ __launch_bounds__(kLutThreads) void k_gemv_lut(const uint32_t* __restrict__ packed,
                                                         const float* __restrict__ gamma,
                                                         const int8_t* __restrict__ xq,
                                                         const float* __restrict__ absmax,
                                                         int N, int K, float* __restrict__ y,
                                                         int32_t* __restrict__ acc_out) {
  __shared__ __align__(16) short tab[kLutWords * kLutWordStride];
  __shared__ int part[kLutWaves][16];
  const int tok = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane & 3;
  const int row = blockIdx.x * 16 + (lane >> 2);
  const int K16 = K >> 4;
  const uint32_t* wrow = packed + (int64_t)(row < N ? row : N - 1) * K16;
  const int8_t* x = xq + (int64_t)tok * K;

  int sum = 0;
  for (int k0 = 0; k0 < K; k0 += kLutK) {
    const int words = min(kLutK, K - k0) >> 4;   // packed words of this chunk
    const int w_base = k0 >> 4;
    // activation pairs of this thread's table groups (group = word * 8 + 2i + h)
    int xa[kLutGroups], xb[kLutGroups];
#pragma unroll
    for (int u = 0; u < kLutGroups; ++u) {
      const int grp = tid + u * kLutThreads;
      const int wl = grp >> 3, i = (grp >> 1) & 3, h = grp & 1;
      const int ka = k0 + 16 * wl + 8 * h + i;
      const bool ok = wl < words;
      xa[u] = ok ? x[ka] : 0;
      xb[u] = ok ? x[ka + 4] : 0;
    }
    // this lane's weight words: of the chunk's 16-byte vectors, this wave
    // takes m = wave * kLutVecs ...; the four lanes of a row take 4m .. 4m + 3
    uint32_t wv[kLutVecs][4];
#pragma unroll
    for (int mm = 0; mm < kLutVecs; ++mm) {
      const int m = wave * kLutVecs + mm;
      const int w0 = 4 * (sub + 4 * m);
      if constexpr (VEC4) {
        const uint4 v = w0 < words ? *reinterpret_cast<const uint4*>(wrow + w_base + w0)
                                   : make_uint4(0, 0, 0, 0);
        wv[mm][0] = v.x; wv[mm][1] = v.y; wv[mm][2] = v.z; wv[mm][3] = v.w;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) wv[mm][q] = w0 + q < words ? wrow[w_base + w0 + q] : 0u;
      }
    }
    lds_sync();   // the previous chunk's lookups are done
#pragma unroll
    for (int u = 0; u < kLutGroups; ++u) {
      const int grp = tid + u * kLutThreads;
      const int wl = grp >> 3;
      if (wl >= words) continue;
      short* t = tab + wl * kLutWordStride + (grp & 7) * 16;
      // entry ca + 4 cb; codes 0, 1, 2 stand for -1, 0, +1, code 3 never occurs
      const int a = xa[u], b = xb[u];
      const int va[4] = {-a, 0, a, 0};
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int vb = cb == 0 ? -b : cb == 1 ? 0 : cb == 2 ? b : 0;
        const bool dead = cb == 3;
        const int e0 = dead ? 0 : va[0] + vb, e1 = dead ? 0 : va[1] + vb;
        const int e2 = dead ? 0 : va[2] + vb;
        // entries 4cb .. 4cb + 3 as two dwords of int16 pairs (8-byte aligned)
        uint2 pr;
        pr.x = (uint32_t)(e0 & 0xffff) | ((uint32_t)e1 << 16);
        pr.y = (uint32_t)(e2 & 0xffff);
        *reinterpret_cast<uint2*>(t + 4 * cb) = pr;
      }
    }
    lds_sync();
    // lookups: one per nibble, words past the chunk skipped
#pragma unroll
    for (int mm = 0; mm < kLutVecs; ++mm) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int wl = 4 * (sub + 4 * (wave * kLutVecs + mm)) + q;
        if (wl >= words) continue;
        const uint32_t w = wv[mm][q];
        const short* t = tab + wl * kLutWordStride;
#pragma unroll
        for (int p = 0; p < 8; ++p) sum += t[p * 16 + ((w >> (4 * p)) & 15)];
      }
    }
  }
  // the four lanes of a row, then the four waves
  sum += __shfl_xor(sum, 1);
  sum += __shfl_xor(sum, 2);
  if (sub == 0) part[wave][lane >> 2] = sum;
  lds_sync();
  if (wave == 0 && lane < 16) {
    const int r = blockIdx.x * 16 + lane;
    if (r < N) {
      const int s = part[0][lane] + part[1][lane] + part[2][lane] + part[3][lane];
      const int64_t o = (int64_t)tok * N + r;
      if (acc_out) acc_out[o] = s;
      y[o] = (float)s * out_scale(gamma[0], absmax[tok]);
    }
  }
}

}  // namespace

hipError_t launch_gemv_lut(const uint8_t* packed, const float* gamma, const int8_t* xq,
                           const float* absmax, int64_t t, int64_t n, int64_t k, float* y,
                           int32_t* acc, hipStream_t stream) {
  const bool vec4 = (k % 64) == 0 && (reinterpret_cast<uintptr_t>(packed) % 16) == 0;
  const unsigned bx = (unsigned)((n + 15) / 16);
  const uint32_t* pw = reinterpret_cast<const uint32_t*>(packed);
  for (int64_t t0 = 0; t0 < t; t0 += 65535) {
    const dim3 grid(bx, (unsigned)(t - t0 < 65535 ? t - t0 : 65535));
    const int8_t* xs = xq + t0 * k;
    float* ys = y + t0 * n;
    int32_t* as = acc ? acc + t0 * n : nullptr;
    const int ni = (int)n, ki = (int)k;
    if (vec4)
      k_gemv_lut<true><<<grid, kLutThreads, 0, stream>>>(pw, gamma, xs, absmax + t0, ni, ki, ys, as);
    else
      k_gemv_lut<false><<<grid, kLutThreads, 0, stream>>>(pw, gamma, xs, absmax + t0, ni, ki, ys, as);
  }
  return hipGetLastError();
}

}  // namespace bl
