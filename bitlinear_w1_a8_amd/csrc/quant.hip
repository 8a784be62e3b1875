// Step A1: per-token absmax quantisation of activations to int8.
//
// "BitNet解读" (markgoyens.top), activation quantisation: every token is
// scaled into [-Qb, Qb] without a zero point; the 2B4T report, section 2,
// takes the absmax per token and uses 8 bits.  Per row: a = max |x|,
// s = 127 / max(a, eps) (IEEE binary32 division), q = clamp(rne(x * s)).
//
// One block per token row.  The row is read once into registers (up to
// kMaxVec 16-byte vectors per thread), the absmax is reduced with DPP row
// operations inside each wave and across waves through LDS, and the same
// registers are then scaled, rounded, clipped and stored as int8.
#include "bl_internal.h"

namespace bl {
namespace {

constexpr int kMaxVec = 8;      // 16-byte vectors held per thread
constexpr int kMaxWaves = 16;   // up to 1024 threads per row

// DPP controls (GCN/CDNA encoding).
constexpr int kQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Max over the 16 lanes of each DPP row, result in every lane of the row.
__device__ __forceinline__ int row_max_u(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(0, v, kQuadSwap1, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, kQuadSwap2, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, kRowHalfMirror, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, kRowMirror, 0xF, 0xF, false));
  return v;
}

__device__ __forceinline__ int row_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, kQuadSwap1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kQuadSwap2, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kRowHalfMirror, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kRowMirror, 0xF, 0xF, false);
  return v;
}

// Whole-wave results, uniform across the wave: combine the four rows.
__device__ __forceinline__ int wave_max_u(int v) {
  v = row_max_u(v);
  const int a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const int c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

__device__ __forceinline__ int wave_sum(int v) {
  v = row_sum(v);
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
         __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

// Element access for the two input dtypes; a 16-byte vector holds E elements.
template <int BF16> struct In;
template <> struct In<0> {
  static constexpr int E = 4;
  __device__ static float get(const uint4& v, int i) {
    const uint32_t w = i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
    return __uint_as_float(w);
  }
};
template <> struct In<1> {
  static constexpr int E = 8;
  __device__ static float get(const uint4& v, int i) {
    const uint32_t w = (i >> 1) == 0 ? v.x : (i >> 1) == 1 ? v.y : (i >> 1) == 2 ? v.z : v.w;
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));  // exact widening
  }
};

__device__ __forceinline__ int quant1(float x, float s) {
  const float v = x * s;  // one binary32 product
  return (int)fminf(fmaxf(rintf(v), -kQb), kQb);
}

template <int BF16>
__device__ __forceinline__ void quant_store(const uint4& v, float s, int8_t* dst, int& sum) {
  constexpr int E = In<BF16>::E;
  uint32_t out[E / 4];
#pragma unroll
  for (int w = 0; w < E / 4; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int q = quant1(In<BF16>::get(v, w * 4 + b), s);
      sum += q;
      word |= (uint32_t)(q & 0xff) << (8 * b);
    }
    out[w] = word;
  }
  if (E == 8) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(out[0], out[E / 4 - 1]);
  } else {
    *reinterpret_cast<uint32_t*>(dst) = out[0];
  }
}

template <int BF16>
__device__ __forceinline__ int vec_absmax_bits(const uint4& v) {
  int m = 0;
#pragma unroll
  for (int i = 0; i < In<BF16>::E; ++i)
    m = max(m, (int)(__float_as_uint(In<BF16>::get(v, i)) & 0x7fffffffu));
  return m;  // non-negative binary32 bit patterns order like their values
}

template <int BF16>
__global__ __launch_bounds__(1024) void k_act_quant(const uint4* __restrict__ x, int k,
                                                    int8_t* __restrict__ xq,
                                                    float* __restrict__ absmax,
                                                    int32_t* __restrict__ rowsum) {
  constexpr int E = In<BF16>::E;
  __shared__ int red[kMaxWaves];
  __shared__ int red2[kMaxWaves];
  const int nvec = k / E;
  const int64_t row = blockIdx.x;
  const uint4* xr = x + row * (int64_t)nvec;
  int8_t* qr = xq + row * (int64_t)k;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int lane = tid & 63, wave = tid >> 6, nwaves = nthr >> 6;

  uint4 v[kMaxVec];
  int m = 0;
#pragma unroll
  for (int i = 0; i < kMaxVec; ++i) {
    const int idx = tid + i * nthr;
    if (idx < nvec) {
      v[i] = xr[idx];
      m = max(m, vec_absmax_bits<BF16>(v[i]));
    }
  }
  for (int idx = tid + kMaxVec * nthr; idx < nvec; idx += nthr)
    m = max(m, vec_absmax_bits<BF16>(xr[idx]));

  m = wave_max_u(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  int mb = red[0];
  for (int wv = 1; wv < nwaves; ++wv) mb = max(mb, red[wv]);
  const float a = __uint_as_float((uint32_t)mb);
  const float s = kQb / fmaxf(a, kEps);  // IEEE binary32 division

  int sum = 0;
#pragma unroll
  for (int i = 0; i < kMaxVec; ++i) {
    const int idx = tid + i * nthr;
    if (idx < nvec) quant_store<BF16>(v[i], s, qr + (int64_t)idx * E, sum);
  }
  for (int idx = tid + kMaxVec * nthr; idx < nvec; idx += nthr)
    quant_store<BF16>(xr[idx], s, qr + (int64_t)idx * E, sum);

  if (rowsum) {
    sum = wave_sum(sum);
    if (lane == 0) red2[wave] = sum;
    __syncthreads();
    if (tid == 0) {
      int t = 0;
      for (int wv = 0; wv < nwaves; ++wv) t += red2[wv];
      rowsum[row] = t;
    }
  }
  if (tid == 0) absmax[row] = a;
}

}  // namespace

hipError_t launch_quant(const void* x, int bf16, int64_t t, int64_t k, int8_t* xq,
                        float* absmax, int32_t* rowsum, hipStream_t stream) {
  const int e = bf16 ? 8 : 4;
  const int64_t nvec = k / e;
  // enough threads that each holds at most kMaxVec vectors, in whole waves
  int64_t thr = (nvec + kMaxVec - 1) / kMaxVec;
  thr = ((thr + 63) / 64) * 64;
  if (thr < 64) thr = 64;
  if (thr > 64 * kMaxWaves) thr = 64 * kMaxWaves;
  const dim3 grid((unsigned)t), block((unsigned)thr);
  if (bf16)
    k_act_quant<1><<<grid, block, 0, stream>>>(static_cast<const uint4*>(x), (int)k, xq, absmax,
                                               rowsum);
  else
    k_act_quant<0><<<grid, block, 0, stream>>>(static_cast<const uint4*>(x), (int)k, xq, absmax,
                                               rowsum);
  return hipGetLastError();
}

}  // namespace bl
