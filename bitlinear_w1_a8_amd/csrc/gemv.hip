// Steps A2 + A3 for few tokens (decode): stream the 2-bit packed weights from
// HBM once, unpack them in registers, contract with int8 activations on the
// matrix cores, rescale in the epilogue.
//
// The 2B4T report (section 5.1, GPU inference) keeps four ternary weights per
// byte in HBM, moves them on chip, unpacks them and multiplies with 8-bit
// activations; "BitNet解读" (computational efficiency) notes that weight
// traffic from DRAM, not arithmetic, bounds this step.  Here the unpack is two
// VALU operations per four weights and stays in registers:
//   codes = (word >> 2j) & 0x03030303
// gives the codes c = t + 1 of 16 consecutive k as four int8 dwords, already
// in k order, which is an MFMA operand as it stands.  The MFMA then sums
// c * q = (t + 1) * q; subtracting the token's sum of q over the same k
// (computed here from the same activation bytes) leaves the exact sum t * q.
//
// MFMA v_mfma_i32_16x16x64_i8: A = 16 weight rows x 64 k, B = 64 k x 16 tokens.
// Lane l = 16*qg + r feeds A row r and B column r with the 16 k of group qg;
// because A and B take k from the same (lane group, byte) positions, any
// k order inside an MFMA gives the same sum.  The 16x16 result sits in lane l
// as rows 4*qg + {0..3} of column r.
//
// Work split: a block owns 16*RT weight rows; its waves split K into chunks of
// 64*VEC k; partial 16x16 tiles are summed through LDS; the epilogue
// multiplies by gamma * max(absmax, eps) / 127.
#include "bl_internal.h"

namespace bl {
namespace {

constexpr int kGemvTokens = 64;   // tokens per launch (4 MFMA column tiles)
constexpr int kMaxWaves = 8;

template <int VEC, int RT, int NTT>
__global__ __launch_bounds__(512) void k_gemv(const uint32_t* __restrict__ packed,
                                              const float* __restrict__ gamma,
                                              const int8_t* __restrict__ xq,
                                              const float* __restrict__ absmax, int T, int N,
                                              int K, float* __restrict__ y,
                                              int32_t* __restrict__ acc_out) {
  extern __shared__ int red[];  // [nwaves][RT*NTT*4][64]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int qg = lane >> 4, r = lane & 15;
  const int K16 = K >> 4;                           // packed words per row
  const int nchunks = (K16 + 4 * VEC - 1) / (4 * VEC);
  const int n0 = blockIdx.x * 16 * RT;

  const uint32_t* wrow[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    int n = n0 + 16 * rt + r;
    n = n < N ? n : N - 1;                          // rows past N are computed, never stored
    wrow[rt] = packed + (int64_t)n * K16;
  }
  const int8_t* xrow[NTT];
  bool tvalid[NTT];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    const int tok = 16 * tt + r;
    tvalid[tt] = tok < T;
    xrow[tt] = xq + (int64_t)(tvalid[tt] ? tok : 0) * K;
  }

  v4i acc[RT][NTT];
  int qs[NTT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[rt][tt] = v4i{0, 0, 0, 0};
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) qs[tt] = 0;

  for (int c = wave; c < nchunks; c += nwaves) {
    const int wi = c * 4 * VEC + qg * VEC;          // first packed word of this lane
    const bool kvalid = wi < K16;                   // VEC divides K16 when VEC > 1
    uint32_t wv[RT][VEC];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if constexpr (VEC == 4) {
        const uint4 u =
            kvalid ? *reinterpret_cast<const uint4*>(wrow[rt] + wi) : make_uint4(0, 0, 0, 0);
        wv[rt][0] = u.x; wv[rt][1] = u.y; wv[rt][2] = u.z; wv[rt][3] = u.w;
      } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v) wv[rt][v] = kvalid ? wrow[rt][wi + v] : 0u;
      }
    }
    uint32_t xv[NTT][4 * VEC];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      const bool ok = kvalid && tvalid[tt];
      const uint4* src = reinterpret_cast<const uint4*>(xrow[tt] + (int64_t)wi * 16);
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const uint4 u = ok ? src[v] : make_uint4(0, 0, 0, 0);
        xv[tt][4 * v + 0] = u.x; xv[tt][4 * v + 1] = u.y;
        xv[tt][4 * v + 2] = u.z; xv[tt][4 * v + 3] = u.w;
      }
#pragma unroll
      for (int d = 0; d < 4 * VEC; ++d)
        qs[tt] = __builtin_amdgcn_sdot4((int)xv[tt][d], 0x01010101, qs[tt], false);
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const uint32_t w = wv[rt][v];
        const v4i a = {(int)codes_of(w, 0), (int)codes_of(w, 1), (int)codes_of(w, 2),
                       (int)codes_of(w, 3)};
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
          const v4i b = {(int)xv[tt][4 * v + 0], (int)xv[tt][4 * v + 1], (int)xv[tt][4 * v + 2],
                         (int)xv[tt][4 * v + 3]};
          acc[rt][tt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[rt][tt], 0, 0, 0);
        }
      }
    }
  }

  // sum of q over this wave's k for the token of column r: add the 4 lane groups
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) {
    int s = qs[tt];
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[rt][tt][v] -= s;
  }

  constexpr int kSlots = RT * NTT * 4;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        red[(wave * kSlots + (rt * NTT + tt) * 4 + v) * 64 + lane] = acc[rt][tt][v];
  __syncthreads();

  const float g = gamma[0];
  constexpr int kRows = 16 * RT, kToks = 16 * NTT;
  for (int idx = threadIdx.x; idx < kRows * kToks; idx += blockDim.x) {
    const int nl = idx % kRows, tl = idx / kRows;
    const int n = n0 + nl;
    if (n >= N || tl >= T) continue;
    const int rt = nl >> 4, i = nl & 15, tt = tl >> 4, j = tl & 15;
    const int slot = (rt * NTT + tt) * 4 + (i & 3);
    const int ln = (i >> 2) * 16 + j;
    int s = 0;
    for (int wv = 0; wv < nwaves; ++wv) s += red[(wv * kSlots + slot) * 64 + ln];
    const int64_t o = (int64_t)tl * N + n;
    if (acc_out) acc_out[o] = s;
    y[o] = (float)s * out_scale(g, absmax[tl]);
  }
}

template <int VEC, int RT, int NTT>
void run(const uint8_t* packed, const float* gamma, const int8_t* xq, const float* absmax,
         int t, int n, int k, float* y, int32_t* acc, hipStream_t stream) {
  const int k16 = k / 16;
  const int nchunks = (k16 + 4 * VEC - 1) / (4 * VEC);
  int nw = nchunks / 2;                 // at least two chunks per wave where possible
  if (nw < 1) nw = 1;
  if (nw > kMaxWaves) nw = kMaxWaves;
  const int grid = (n + 16 * RT - 1) / (16 * RT);
  const size_t lds = (size_t)nw * RT * NTT * 4 * 64 * sizeof(int);
  k_gemv<VEC, RT, NTT><<<grid, nw * 64, lds, stream>>>(
      reinterpret_cast<const uint32_t*>(packed), gamma, xq, absmax, t, n, k, y, acc);
}

template <int VEC>
void run_tokens(const uint8_t* packed, const float* gamma, const int8_t* xq,
                const float* absmax, int t, int n, int k, float* y, int32_t* acc,
                hipStream_t stream) {
  if (t <= 16)
    run<VEC, 1, 1>(packed, gamma, xq, absmax, t, n, k, y, acc, stream);
  else if (t <= 32)
    run<VEC, 2, 2>(packed, gamma, xq, absmax, t, n, k, y, acc, stream);
  else
    run<VEC, 2, 4>(packed, gamma, xq, absmax, t, n, k, y, acc, stream);
}

}  // namespace

hipError_t launch_gemv(const uint8_t* packed, const float* gamma, const int8_t* xq,
                       const float* absmax, int64_t t, int64_t n, int64_t k, float* y,
                       int32_t* acc, hipStream_t stream) {
  const bool vec4 = (k % 64) == 0 && (reinterpret_cast<uintptr_t>(packed) % 16) == 0 &&
                    (reinterpret_cast<uintptr_t>(xq) % 16) == 0;
  for (int64_t t0 = 0; t0 < t; t0 += kGemvTokens) {
    const int tc = (int)(t - t0 < kGemvTokens ? t - t0 : kGemvTokens);
    const int8_t* xs = xq + t0 * k;
    float* ys = y + t0 * n;
    int32_t* as = acc ? acc + t0 * n : nullptr;
    if (vec4)
      run_tokens<4>(packed, gamma, xs, absmax + t0, tc, (int)n, (int)k, ys, as, stream);
    else
      run_tokens<1>(packed, gamma, xs, absmax + t0, tc, (int)n, (int)k, ys, as, stream);
  }
  return hipGetLastError();
}

}  // namespace bl
