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
//
// With the sub-layer norm in front (SubLN, read as an RMS norm with a
// per-feature gain g and no bias: 2B4T report section 2, the explainer's
// component table): the per-token absmax scale cancels the per-token RMS
// factor r = 1 / sqrt(mean(x^2) + eps_n), so the codes are those of
// u = x * g (one binary32 product per element) and the token's scale handed
// to the rescale is r * max|u|.  The sum of squares is taken in binary64,
// where every x^2 is exact.
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

// Elements e of a 16-byte vector, widened exactly to binary32, times the gain
// (the sub-layer norm) or as they are.
template <int BF16, bool NORM>
__device__ __forceinline__ void elems(const uint4& v, const float* g, float (&f)[In<BF16>::E]) {
#pragma unroll
  for (int e = 0; e < In<BF16>::E; ++e) f[e] = In<BF16>::get(v, e);
  if constexpr (NORM) {
    const float4* g4 = reinterpret_cast<const float4*>(g);
#pragma unroll
    for (int w = 0; w < In<BF16>::E / 4; ++w) {
      const float4 gv = g4[w];
      f[4 * w] *= gv.x;
      f[4 * w + 1] *= gv.y;
      f[4 * w + 2] *= gv.z;
      f[4 * w + 3] *= gv.w;
    }
  }
}

__device__ __forceinline__ double vec_sumsq(const float* f, int n) {
  double s = 0.0;
  for (int e = 0; e < n; ++e) s += (double)f[e] * (double)f[e];
  return s;
}

__device__ __forceinline__ int quant1(float x, float s) {
  const float v = x * s;  // one binary32 product
  return (int)fminf(fmaxf(rintf(v), -kQb), kQb);
}

template <int BF16, bool NORM>
__device__ __forceinline__ void quant_store(const uint4& v, const float* g, float s, int8_t* dst,
                                            int& sum) {
  constexpr int E = In<BF16>::E;
  float f[E];
  elems<BF16, NORM>(v, g, f);
  uint32_t out[E / 4];
#pragma unroll
  for (int w = 0; w < E / 4; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int q = quant1(f[w * 4 + b], s);
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

// absmax bits of the vector's elements (times the gain); with the norm, also
// adds the squares of the raw elements to ss
template <int BF16, bool NORM>
__device__ __forceinline__ int vec_absmax_bits(const uint4& v, const float* g, double& ss) {
  constexpr int E = In<BF16>::E;
  float f[E];
  elems<BF16, false>(v, g, f);
  if constexpr (NORM) ss += vec_sumsq(f, E);
  elems<BF16, NORM>(v, g, f);
  int m = 0;
#pragma unroll
  for (int i = 0; i < E; ++i) m = max(m, (int)(__float_as_uint(f[i]) & 0x7fffffffu));
  return m;  // non-negative binary32 bit patterns order like their values
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <int BF16, bool NORM>
__global__ __launch_bounds__(1024) void k_act_quant(const uint4* __restrict__ x, int k,
                                                    int8_t* __restrict__ xq,
                                                    float* __restrict__ absmax,
                                                    int32_t* __restrict__ rowsum,
                                                    const float* __restrict__ gain,
                                                    float eps_n) {
  constexpr int E = In<BF16>::E;
  __shared__ int red[kMaxWaves];
  __shared__ int red2[kMaxWaves];
  __shared__ double redss[kMaxWaves];
  const int nvec = k / E;
  const int64_t row = blockIdx.x;
  const uint4* xr = x + row * (int64_t)nvec;
  int8_t* qr = xq + row * (int64_t)k;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int lane = tid & 63, wave = tid >> 6, nwaves = nthr >> 6;

  uint4 v[kMaxVec];
  int m = 0;
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < kMaxVec; ++i) {
    const int idx = tid + i * nthr;
    if (idx < nvec) {
      v[i] = xr[idx];
      m = max(m, vec_absmax_bits<BF16, NORM>(v[i], gain + idx * E, ss));
    }
  }
  for (int idx = tid + kMaxVec * nthr; idx < nvec; idx += nthr)
    m = max(m, vec_absmax_bits<BF16, NORM>(xr[idx], gain + idx * E, ss));

  m = wave_max_u(m);
  if (lane == 0) red[wave] = m;
  if constexpr (NORM) {
    ss = wave_sum_f64(ss);
    if (lane == 0) redss[wave] = ss;
  }
  __syncthreads();
  int mb = red[0];
  for (int wv = 1; wv < nwaves; ++wv) mb = max(mb, red[wv]);
  const float a = __uint_as_float((uint32_t)mb);
  const float s = kQb / fmaxf(a, kEps);  // IEEE binary32 division

  int sum = 0;
#pragma unroll
  for (int i = 0; i < kMaxVec; ++i) {
    const int idx = tid + i * nthr;
    if (idx < nvec) quant_store<BF16, NORM>(v[i], gain + idx * E, s, qr + (int64_t)idx * E, sum);
  }
  for (int idx = tid + kMaxVec * nthr; idx < nvec; idx += nthr)
    quant_store<BF16, NORM>(xr[idx], gain + idx * E, s, qr + (int64_t)idx * E, sum);

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
  if (tid == 0) {
    if constexpr (NORM) {
      double t = redss[0];
      for (int wv = 1; wv < nwaves; ++wv) t += redss[wv];
      const double r = 1.0 / sqrt(t / (double)k + (double)eps_n);
      absmax[row] = (float)((double)a * r);
    } else {
      absmax[row] = a;
    }
  }
}

hipError_t launch_quant_impl(const void* x, int bf16, int64_t t, int64_t k, int8_t* xq,
                             float* absmax, int32_t* rowsum, const float* gain, float eps_n,
                             hipStream_t stream) {
  const int e = bf16 ? 8 : 4;
  const int64_t nvec = k / e;
  // enough threads that each holds at most kMaxVec vectors, in whole waves
  int64_t thr = (nvec + kMaxVec - 1) / kMaxVec;
  thr = ((thr + 63) / 64) * 64;
  if (thr < 64) thr = 64;
  if (thr > 64 * kMaxWaves) thr = 64 * kMaxWaves;
  const dim3 grid((unsigned)t), block((unsigned)thr);
  const uint4* xv = static_cast<const uint4*>(x);
  if (gain) {
    if (bf16)
      k_act_quant<1, true><<<grid, block, 0, stream>>>(xv, (int)k, xq, absmax, rowsum, gain, eps_n);
    else
      k_act_quant<0, true><<<grid, block, 0, stream>>>(xv, (int)k, xq, absmax, rowsum, gain, eps_n);
  } else {
    if (bf16)
      k_act_quant<1, false><<<grid, block, 0, stream>>>(xv, (int)k, xq, absmax, rowsum, gain, eps_n);
    else
      k_act_quant<0, false><<<grid, block, 0, stream>>>(xv, (int)k, xq, absmax, rowsum, gain, eps_n);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant(const void* x, int bf16, int64_t t, int64_t k, int8_t* xq,
                        float* absmax, int32_t* rowsum, hipStream_t stream) {
  return launch_quant_impl(x, bf16, t, k, xq, absmax, rowsum, nullptr, 0.0f, stream);
}

hipError_t launch_subln_quant(const void* x, int bf16, const float* gain, float eps_n, int64_t t,
                              int64_t k, int8_t* xq, float* scale, int32_t* rowsum,
                              hipStream_t stream) {
  return launch_quant_impl(x, bf16, t, k, xq, scale, rowsum, gain, eps_n, stream);
}

}  // namespace bl
