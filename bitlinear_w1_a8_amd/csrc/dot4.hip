// Steps A2 + A3 with packed int8 dot instructions (v_dot4_i32_i8) instead of
// the matrix cores: a second comparison design for the decode path.
//
// Per packed word (16 k of a row: k = 16g + 4j + i at bits 8i + 2j) the codes
// of field j, (w >> 2j) & 0x03030303, are four consecutive k as bytes, and
// one v_dot4 with dword j of the 16 activation bytes of the word adds
// sum c * q over them; subtracting the token's sum of q leaves the exact
// sum t * q ("BitNet解读", computational efficiency: +1 / -1 / 0 turn the
// products into additions, subtractions and skips).  Unpacking costs 7 VALU
// per word here (5 on the matrix-core path, whose masked fields need no
// shift), and every token then needs 4 more VALU per word, where one MFMA
// serves 16 token columns.
//
// Layout: a block owns 16 rows and one token; four lanes share a row and
// read 64 contiguous bytes of it per load; the four waves split each
// 16384-k chunk of the row; the token's int8 activations of the chunk sit in
// LDS (16 KiB).
#include "bl_internal.h"

namespace bl {
namespace {

constexpr int kDotK = 16384;   // k per LDS chunk
constexpr int kDotWaves = 4;

template <bool VEC4>
__global__ __launch_bounds__(kDotWaves * 64) void k_gemv_dot4(const uint32_t* __restrict__ packed,
                                                             const float* __restrict__ gamma,
                                                             const int8_t* __restrict__ xq,
                                                             const float* __restrict__ absmax,
                                                             int N, int K, float* __restrict__ y,
                                                             int32_t* __restrict__ acc_out) {
  __shared__ __align__(16) unsigned char xs[kDotK];
  __shared__ int part[kDotWaves][16];
  __shared__ int qpart[kDotWaves];
  const int tok = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane & 3;
  const int row = blockIdx.x * 16 + (lane >> 2);
  const int K16 = K >> 4;
  const uint32_t* wrow = packed + (int64_t)(row < N ? row : N - 1) * K16;
  const uint4* x4g = reinterpret_cast<const uint4*>(xq + (int64_t)tok * K);

  int sum = 0, qs = 0;
  for (int k0 = 0; k0 < K; k0 += kDotK) {
    const int words = min(kDotK, K - k0) >> 4;      // 16-byte activation vectors = packed words
    const int wb = k0 >> 4;
    __syncthreads();                                 // the previous chunk is no longer read
    for (int i = tid; i < words; i += kDotWaves * 64) {
      const uint4 v = x4g[wb + i];
      reinterpret_cast<uint4*>(xs)[i] = v;
      qs = __builtin_amdgcn_sdot4((int)v.x, 0x01010101, qs, false);
      qs = __builtin_amdgcn_sdot4((int)v.y, 0x01010101, qs, false);
      qs = __builtin_amdgcn_sdot4((int)v.z, 0x01010101, qs, false);
      qs = __builtin_amdgcn_sdot4((int)v.w, 0x01010101, qs, false);
    }
    __syncthreads();
    const uint4* x4 = reinterpret_cast<const uint4*>(xs);
    // wave w takes a quarter of the chunk; the row's four lanes take 16-byte
    // vectors (or words) sub, sub + 4, ... of it (64 contiguous bytes)
    auto word_dot = [&](uint32_t w, int wi) {
      const uint4 xv = x4[wi];
      sum = __builtin_amdgcn_sdot4((int)codes_of(w, 0), (int)xv.x, sum, false);
      sum = __builtin_amdgcn_sdot4((int)codes_of(w, 1), (int)xv.y, sum, false);
      sum = __builtin_amdgcn_sdot4((int)codes_of(w, 2), (int)xv.z, sum, false);
      sum = __builtin_amdgcn_sdot4((int)codes_of(w, 3), (int)xv.w, sum, false);
    };
    if constexpr (VEC4) {
      const int nvec = words >> 2;                   // K % 64 == 0: whole vectors
      const int per = (nvec + kDotWaves - 1) / kDotWaves;
      const int v0 = wave * per, v1 = min(nvec, v0 + per);
      for (int v = v0 + sub; v < v1; v += 4) {
        const uint4 pw = *reinterpret_cast<const uint4*>(wrow + wb + 4 * v);
        word_dot(pw.x, 4 * v);
        word_dot(pw.y, 4 * v + 1);
        word_dot(pw.z, 4 * v + 2);
        word_dot(pw.w, 4 * v + 3);
      }
    } else {
      const int per = (words + kDotWaves - 1) / kDotWaves;
      const int w0 = wave * per, w1 = min(words, w0 + per);
      for (int wi = w0 + sub; wi < w1; wi += 4) word_dot(wrow[wb + wi], wi);
    }
  }
  // the token's sum of q over K (every thread staged part of it)
  for (int o = 32; o > 0; o >>= 1) qs += __shfl_xor(qs, o);
  if (lane == 0) qpart[wave] = qs;
  sum += __shfl_xor(sum, 1);
  sum += __shfl_xor(sum, 2);
  if (sub == 0) part[wave][lane >> 2] = sum;
  __syncthreads();
  if (wave == 0 && lane < 16) {
    const int r = blockIdx.x * 16 + lane;
    if (r < N) {
      const int q = qpart[0] + qpart[1] + qpart[2] + qpart[3];
      const int s = part[0][lane] + part[1][lane] + part[2][lane] + part[3][lane] - q;
      const int64_t o = (int64_t)tok * N + r;
      if (acc_out) acc_out[o] = s;
      y[o] = (float)s * out_scale(gamma[0], absmax[tok]);
    }
  }
}

}  // namespace

hipError_t launch_gemv_dot4(const uint8_t* packed, const float* gamma, const int8_t* xq,
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
    if (vec4)
      k_gemv_dot4<true><<<grid, kDotWaves * 64, 0, stream>>>(pw, gamma, xs, absmax + t0, (int)n,
                                                             (int)k, ys, as);
    else
      k_gemv_dot4<false><<<grid, kDotWaves * 64, 0, stream>>>(pw, gamma, xs, absmax + t0, (int)n,
                                                              (int)k, ys, as);
  }
  return hipGetLastError();
}

}  // namespace bl
