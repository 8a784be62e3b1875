// Step A1: per-token absmax quantisation of activations to int8.
//
// "BitNet解读" (markgoyens.top), activation quantisation: every token is
// scaled into [-Qb, Qb] without a zero point; the 2B4T report, section 2,
// takes the absmax per token and uses 8 bits.  Per row: a = max |x|,
// s = 127 / max(a, eps) (IEEE binary32 division), q = clamp(rne(x * s)).
//
// One block per token row.  The row is read once into registers (up to
// kQuantVpt 16-byte vectors per thread), the absmax is reduced with DPP row
// operations inside each wave and across waves through LDS, and the same
// registers are then scaled, rounded, clipped and stored as int8.
//
// The sub-layer norm in front of it (SubLN, read as an RMS norm with a
// per-feature gain g and no bias: 2B4T report section 2, the explainer's
// component table) runs in its own kernel, k_subln_quant: normalise, then
// quantise the normalised row, with the sum of squares taken exactly.
#include "bl_internal.h"

namespace bl {
namespace {

constexpr int kMaxWaves = 16;   // up to 1024 threads per row
constexpr int kSublnRegs = 4;   // 16-byte vectors of the row SubLN holds per thread
constexpr int kQuantVpt = 4;    // vectors per thread of the act-quant launch, held in registers
                                // (longer rows read the rest again); 64 VGPRs, eight waves per SIMD

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

// Elements of a 16-byte vector, widened exactly to binary32.
template <int BF16>
__device__ __forceinline__ void elems(const uint4& v, float (&f)[In<BF16>::E]) {
#pragma unroll
  for (int e = 0; e < In<BF16>::E; ++e) f[e] = In<BF16>::get(v, e);
}

// The same elements times the gain (one binary32 product each): u = x * g.
template <int BF16>
__device__ __forceinline__ void elems_gain(const uint4& v, const float* g,
                                           float (&f)[In<BF16>::E]) {
  elems<BF16>(v, f);
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

__device__ __forceinline__ int quant1(float x, float s) {
  const float v = x * s;  // one binary32 product
  return (int)fminf(fmaxf(rintf(v), -kQb), kQb);
}

// Codes of E values, stored as E bytes at dst (8-byte or 4-byte aligned).
template <int E>
__device__ __forceinline__ void quant_store_f(const float (&f)[E], float s, int8_t* dst, int& sum) {
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

template <int BF16>
__device__ __forceinline__ void quant_store(const uint4& v, float s, int8_t* dst, int& sum) {
  float f[In<BF16>::E];
  elems<BF16>(v, f);
  quant_store_f(f, s, dst, sum);
}

// Largest |f| of the E values as a binary32 bit pattern (non-negative
// patterns order like their values).
template <int E>
__device__ __forceinline__ int absmax_bits(const float (&f)[E]) {
  int m = 0;
#pragma unroll
  for (int i = 0; i < E; ++i) m = max(m, (int)(__float_as_uint(f[i]) & 0x7fffffffu));
  return m;
}

template <int BF16>
__device__ __forceinline__ int vec_absmax_bits(const uint4& v) {
  float f[In<BF16>::E];
  elems<BF16>(v, f);
  return absmax_bits(f);
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

  uint4 v[kQuantVpt];
  int m = 0;
#pragma unroll
  for (int i = 0; i < kQuantVpt; ++i) {
    const int idx = tid + i * nthr;
    if (idx < nvec) {
      v[i] = xr[idx];
      m = max(m, vec_absmax_bits<BF16>(v[i]));
    }
  }
  for (int idx = tid + kQuantVpt * nthr; idx < nvec; idx += nthr)
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
  for (int i = 0; i < kQuantVpt; ++i) {
    const int idx = tid + i * nthr;
    if (idx < nvec) quant_store<BF16>(v[i], s, qr + (int64_t)idx * E, sum);
  }
  for (int idx = tid + kQuantVpt * nthr; idx < nvec; idx += nthr)
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

// ------------------------------------------------------------------ SubLN + A1
//
// Per token: S = sum_k x^2 exactly (rounded once to binary64), ms =
// RN32(RN64(S / K)), r = RN32(1 / RN32(sqrt(RN32(ms + eps_n)))), x_hat =
// RN32(RN32(x * g) * r), then step A1 on x_hat; scale[t] = max |x_hat|.
//
// The exact sum.  Let E be the exponent field of the row's largest |x| and
// d = E - e for an element with exponent field e (e = 1 for subnormals and
// zero).  The first pass also finds the smallest nonzero |x|; when every
// nonzero element has d <= 31 (ordinary data) each lane adds its squares
// exactly in fixed point at the row's exponent:
//  - binary32 input, x = m * 2^(e-150) with a 24-bit m: m^2 << (62 - 2d)
//    into a 128-bit integer (fewer than 2^17 terms below 2^110), branch-free;
//  - bf16 input, x = m * 2^(e-134) with an 8-bit m: x^2 by binary64 FMAs
//    into one of two accumulators, d <= 15 (a multiple of 2^(2E-298)) and
//    16 <= d <= 31 (a multiple of 2^(2E-330)).  Each square is below 2^46 of
//    its window's units and a lane adds at most 128 of them (K <= 131072
//    over at most 1024 lanes), so every partial sum is a multiple of the
//    unit below 2^53 units and each FMA is exact; the two sums are then
//    scaled to integers by powers of two.  A lane whose own smallest
//    nonzero |x| has d <= 15 (nearly every lane) uses the first only and
//    tests nothing per element.
// The lanes' sums go to 128 bits in units of 2^(2E-362), are added across
// the wave, and one thread adds the waves' sums in 192 bits and rounds the
// total once to binary64.  A row with a nonzero element more than 31
// binades below its largest (none in ordinary data) instead sums every
// element into per-exponent LDS buckets and rounds their 576-bit total.
//
// max |x_hat| is RN32(max |u| * r): rounding is monotonic, so the largest
// |u| gives the largest |x_hat|.

constexpr int kSqShift = 62;       // bit of m^2 for an element at the row's exponent
constexpr int kSqWindow = 31;      // binades below the largest that the fixed point holds
constexpr int kSqLimbs = 18;       // 576 bits: sums below 2^17 * 2^256 in units of 2^-298
// a lane's bf16 squares: at most 128, each below 2^46, stay below 2^53
static_assert(8 * (kSublnRegs > BITLINEAR_MAX_K / 8 / (64 * kMaxWaves)
                       ? kSublnRegs : BITLINEAR_MAX_K / 8 / (64 * kMaxWaves)) <= 128,
              "bf16 squares per lane");

struct U128 {
  unsigned long long lo, hi;
};

__device__ __forceinline__ void u128_add(U128& a, unsigned long long lo, unsigned long long hi) {
  const unsigned long long l = a.lo + lo;
  a.hi += hi + (l < lo ? 1ull : 0ull);
  a.lo = l;
}

// Significand and effective exponent of |x| (subnormals: e = 1, no hidden bit).
__device__ __forceinline__ void split_f32(float x, uint32_t& m, int& e) {
  const uint32_t b = __float_as_uint(x) & 0x7fffffffu;
  e = (int)(b >> 23);
  m = b & 0x7fffffu;
  if (e) m |= 0x800000u; else e = 1;
}

// Smallest (|x| bits - 1) over the elements, unsigned: 0xffffffff when all are zero.
template <int E>
__device__ __forceinline__ uint32_t minnz_bits_m1(const float (&f)[E], uint32_t m) {
#pragma unroll
  for (int i = 0; i < E; ++i) m = min(m, (__float_as_uint(f[i]) & 0x7fffffffu) - 1u);
  return m;
}

// binary32 input: adds x^2 to the lane's 128-bit sum at the row's exponent
// field ew.  Nonzero elements lie within kSqWindow binades of it; a zero
// adds nothing whatever its shift.
__device__ __forceinline__ void add_square(U128& acc, float x, int ew) {
  uint32_t m;
  int e;
  split_f32(x, m, e);
  const int sh = max(2 * (e - ew) + kSqShift, 0);
  const unsigned long long sq = (unsigned long long)m * m;
  u128_add(acc, sq << sh, (sq >> 1) >> (63 - sh));
}

// bf16 input: x^2 into a (d <= 15) or into b (16 <= d <= 31); thr =
// 2^(ew - 142), the smallest |x| with d <= 15 (0 when every element has it).
// Each square is exact in binary64, and every partial sum is a multiple of
// its window's unit below 2^53 of them, so each FMA is exact.
__device__ __forceinline__ void add_square_bf16(double& a, double& b, float x, float thr) {
  const bool near = fabsf(x) >= thr;
  const double xa = (double)(near ? x : 0.0f), xb = (double)(near ? 0.0f : x);
  a = fma(xa, xa, a);
  b = fma(xb, xb, b);
}

__device__ __forceinline__ U128 wave_sum_u128(U128 a) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const unsigned long long lo = __shfl_xor(a.lo, o), hi = __shfl_xor(a.hi, o);
    u128_add(a, lo, hi);
  }
  return a;
}

template <int BF16>
__global__ __launch_bounds__(1024) void k_subln_quant(const uint4* __restrict__ x, int k,
                                                      const float* __restrict__ gain,
                                                      float eps_n, int8_t* __restrict__ xq,
                                                      float* __restrict__ scale,
                                                      int32_t* __restrict__ rowsum) {
  constexpr int E = In<BF16>::E;
  __shared__ unsigned long long red_lo[kMaxWaves], red_hi[kMaxWaves];
  __shared__ int red_e[kMaxWaves], red_umax[kMaxWaves], red_nz[kMaxWaves], red2[kMaxWaves];
  __shared__ float sh_r, sh_s;
  __shared__ unsigned long long far_hist[2][256];   // per-exponent buckets (rare rows)
  __shared__ uint32_t far_limb[kSqLimbs];            // their exact total (rare rows)
  const int nvec = k / E;
  const int64_t row = blockIdx.x;
  const uint4* xr = x + row * (int64_t)nvec;
  int8_t* qr = xq + row * (int64_t)k;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int lane = tid & 63, wave = tid >> 6, nwaves = nthr >> 6;

  // 1. the row in registers; largest |x| and |u| = |x * g|, smallest nonzero |x|
  uint4 v[kSublnRegs];
  int mx = 0, mu = 0;
  uint32_t nz = 0xffffffffu;
#pragma unroll
  for (int i = 0; i < kSublnRegs; ++i) {
    const int idx = tid + i * nthr;
    if (idx < nvec) {
      v[i] = xr[idx];
      float f[E];
      elems<BF16>(v[i], f);
      mx = max(mx, absmax_bits(f));
      nz = minnz_bits_m1(f, nz);
      elems_gain<BF16>(v[i], gain + idx * E, f);
      mu = max(mu, absmax_bits(f));
    }
  }
  for (int idx = tid + kSublnRegs * nthr; idx < nvec; idx += nthr) {
    float f[E];
    elems<BF16>(xr[idx], f);
    mx = max(mx, absmax_bits(f));
    nz = minnz_bits_m1(f, nz);
    elems_gain<BF16>(xr[idx], gain + idx * E, f);
    mu = max(mu, absmax_bits(f));
  }
  // signed max of 0x7fffffff - nz picks the smallest nz (all-zero lanes: INT_MIN)
  mx = wave_max_u(mx);
  mu = wave_max_u(mu);
  const int nzk = wave_max_u((int)(0x7fffffffu - nz));
  if (lane == 0) {
    red_e[wave] = mx;
    red_umax[wave] = mu;
    red_nz[wave] = nzk;
  }
  __syncthreads();
  int bmx = 0, bnz = INT_MIN;
  for (int wv = 0; wv < nwaves; ++wv) {
    bmx = max(bmx, red_e[wv]);
    bnz = max(bnz, red_nz[wv]);
  }
  const int ew = max(bmx >> 23, 1);             // exponent field of the row's largest |x|
  const uint32_t nzb = 0x7fffffffu - (uint32_t)bnz + 1u;   // smallest nonzero |x| bits (0: none)
  const bool far = nzb != 0u && ew - max((int)(nzb >> 23), 1) > kSqWindow;   // block-uniform

  if (!far) {
    // 2. exact sum of squares, per lane at the row's exponent
    U128 acc;
    if constexpr (BF16) {
      // a lane whose smallest nonzero |x| lies within 15 binades of the row's
      // largest (nearly every lane of ordinary data) needs no window test
      const uint32_t lnz = nz + 1u;              // this lane's smallest nonzero |x| bits, 0: none
      const bool lane_near = lnz == 0u || ew - max((int)(lnz >> 23), 1) <= 15;
      double sa = 0.0, sb = 0.0;
      if (lane_near) {
#pragma unroll
        for (int i = 0; i < kSublnRegs; ++i) {
          const int idx = tid + i * nthr;
          if (idx < nvec) {
            float f[E];
            elems<BF16>(v[i], f);
#pragma unroll
            for (int e = 0; e < E; ++e) {
              const double xd = (double)f[e];
              sa = fma(xd, xd, sa);
            }
          }
        }
        for (int idx = tid + kSublnRegs * nthr; idx < nvec; idx += nthr) {
          float f[E];
          elems<BF16>(xr[idx], f);
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const double xd = (double)f[e];
            sa = fma(xd, xd, sa);
          }
        }
      } else {
        const float thr = ew > 16 ? __uint_as_float((uint32_t)(ew - 15) << 23) : 0.0f;
#pragma unroll
        for (int i = 0; i < kSublnRegs; ++i) {
          const int idx = tid + i * nthr;
          if (idx < nvec) {
            float f[E];
            elems<BF16>(v[i], f);
#pragma unroll
            for (int e = 0; e < E; ++e) add_square_bf16(sa, sb, f[e], thr);
          }
        }
        for (int idx = tid + kSublnRegs * nthr; idx < nvec; idx += nthr) {
          float f[E];
          elems<BF16>(xr[idx], f);
#pragma unroll
          for (int e = 0; e < E; ++e) add_square_bf16(sa, sb, f[e], thr);
        }
      }
      // scaled to integers: a in units of 2^(2 ew - 298) = 2^64 units, b in
      // 2^(2 ew - 330) = 2^32 units (exact power-of-two products)
      const unsigned long long ia =
          (unsigned long long)(sa * __hiloint2double((1321 - 2 * ew) << 20, 0));   // 2^(2(149 - ew))
      const unsigned long long ib =
          (unsigned long long)(sb * __hiloint2double((1353 - 2 * ew) << 20, 0));   // 2^(2(165 - ew))
      acc.lo = ib << 32;
      acc.hi = ia + (ib >> 32);
    } else {
      acc = {0ull, 0ull};
#pragma unroll
      for (int i = 0; i < kSublnRegs; ++i) {
        const int idx = tid + i * nthr;
        if (idx < nvec) {
          float f[E];
          elems<BF16>(v[i], f);
#pragma unroll
          for (int e = 0; e < E; ++e) add_square(acc, f[e], ew);
        }
      }
      for (int idx = tid + kSublnRegs * nthr; idx < nvec; idx += nthr) {
        float f[E];
        elems<BF16>(xr[idx], f);
#pragma unroll
        for (int e = 0; e < E; ++e) add_square(acc, f[e], ew);
      }
    }
    acc = wave_sum_u128(acc);
    if (lane == 0) {
      red_lo[wave] = acc.lo;
      red_hi[wave] = acc.hi;
    }
  } else {
    // rare: every element into per-exponent buckets (m^2 in 24-bit halves),
    // the row read again
    for (int j = tid; j < 512; j += nthr) (&far_hist[0][0])[j] = 0ull;
    __syncthreads();
    for (int idx = tid; idx < nvec; idx += nthr) {
      float f[E];
      elems<BF16>(xr[idx], f);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        uint32_t m;
        int ex;
        split_f32(f[e], m, ex);
        if (m) {
          const unsigned long long sq = (unsigned long long)m * m;
          atomicAdd(&far_hist[0][ex], sq >> 24);
          atomicAdd(&far_hist[1][ex], sq & 0xffffffull);
        }
      }
    }
  }
  __syncthreads();

  // 3. one thread: the exact sum, r, the absmax of x_hat and the step-A1 scale
  if (tid == 0) {
    int um = 0;
    for (int wv = 0; wv < nwaves; ++wv) um = max(um, red_umax[wv]);
    double ssum;
    if (!far) {
      // the waves' sums, all in units of 2^(2 ew - 362), added in 192 bits
      // (at most 16 sums below 2^127 each)
      unsigned long long s0 = 0, s1 = 0, s2 = 0;
      for (int wv = 0; wv < nwaves; ++wv) {
        const unsigned long long lo = red_lo[wv], hi = red_hi[wv];
        const unsigned long long a0 = s0 + lo;
        const unsigned long long c0 = a0 < lo ? 1ull : 0ull;
        const unsigned long long b1 = hi + c0;
        const unsigned long long c1 = b1 < c0 ? 1ull : 0ull;
        const unsigned long long a1 = s1 + b1;
        s2 += c1 + (a1 < b1 ? 1ull : 0ull);
        s0 = a0;
        s1 = a1;
      }
      ssum = u192_to_f64(s0, s1, s2, 2 * ew - 362);
    } else {
      // the buckets in 576 bits in units of 2^-298 (in LDS: an array
      // indexed at run time would take scratch memory)
      uint32_t (&limb)[kSqLimbs] = far_limb;
      for (int i = 0; i < kSqLimbs; ++i) limb[i] = 0;
      for (int ex = 1; ex < 255; ++ex) {   // m^2 = hi * 2^24 + lo, at 2^(2 ex - 300)
        limbs_add(limb, far_hist[0][ex], 2 * ex + 22);
        limbs_add(limb, far_hist[1][ex], 2 * ex - 2);
      }
      ssum = limbs_to_f64(limb, -298);
    }
    const float ms = (float)(ssum / (double)k);   // binary64 mean, one rounding to binary32
    const float root = sqrtf(ms + eps_n);          // binary32 add; correctly rounded root
    const float r = 1.0f / root;                   // IEEE binary32 division
    const float a = __uint_as_float((uint32_t)um) * r;   // = max |x_hat|
    sh_r = r;
    sh_s = kQb / fmaxf(a, kEps);
    scale[row] = a;
  }
  __syncthreads();
  const float r = sh_r, s = sh_s;

  // 4. x_hat = RN32(u * r), quantised with step A1's scale
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kSublnRegs; ++i) {
    const int idx = tid + i * nthr;
    if (idx < nvec) {
      float f[E];
      elems_gain<BF16>(v[i], gain + idx * E, f);
#pragma unroll
      for (int e = 0; e < E; ++e) f[e] *= r;
      quant_store_f(f, s, qr + (int64_t)idx * E, sum);
    }
  }
  for (int idx = tid + kSublnRegs * nthr; idx < nvec; idx += nthr) {
    float f[E];
    elems_gain<BF16>(xr[idx], gain + idx * E, f);
#pragma unroll
    for (int e = 0; e < E; ++e) f[e] *= r;
    quant_store_f(f, s, qr + (int64_t)idx * E, sum);
  }
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
}

// Threads for a row of k elements, e per vector, so that each holds about
// vpt (at most the kernel's register vectors) vectors, in whole waves; beyond 1024 threads the loops
// past the register-held vectors take the rest.
dim3 row_block(int64_t k, int e, int vpt) {
  const int64_t nvec = k / e;
  int64_t thr = (nvec + vpt - 1) / vpt;
  thr = ((thr + 63) / 64) * 64;
  if (thr < 64) thr = 64;
  if (thr > 64 * kMaxWaves) thr = 64 * kMaxWaves;
  return dim3((unsigned)thr);
}

// SubLN does more arithmetic per element than act-quant: 4 vectors per
// thread, or 2 where that leaves the launch below two waves per SIMD (t rows
// of blockDim / 64 waves against 1024 SIMDs), so short launches spread each
// row over more waves.
int subln_vpt(int64_t t, int64_t k, int e) {
  int vpt = kSublnRegs;
  while (vpt > 2 && t * (int64_t)(row_block(k, e, vpt).x / 64) < 2048) vpt /= 2;
  return vpt;
}

}  // namespace

hipError_t launch_quant(const void* x, int bf16, int64_t t, int64_t k, int8_t* xq,
                        float* absmax, int32_t* rowsum, hipStream_t stream) {
  const dim3 grid((unsigned)t), block = row_block(k, bf16 ? 8 : 4, kQuantVpt);
  const uint4* xv = static_cast<const uint4*>(x);
  if (bf16)
    k_act_quant<1><<<grid, block, 0, stream>>>(xv, (int)k, xq, absmax, rowsum);
  else
    k_act_quant<0><<<grid, block, 0, stream>>>(xv, (int)k, xq, absmax, rowsum);
  return hipGetLastError();
}

hipError_t launch_subln_quant(const void* x, int bf16, const float* gain, float eps_n, int64_t t,
                              int64_t k, int8_t* xq, float* scale, int32_t* rowsum,
                              hipStream_t stream) {
  const int e = bf16 ? 8 : 4;
  const dim3 grid((unsigned)t), block = row_block(k, e, subln_vpt(t, k, e));
  const uint4* xv = static_cast<const uint4*>(x);
  if (bf16)
    k_subln_quant<1><<<grid, block, 0, stream>>>(xv, (int)k, gain, eps_n, xq, scale, rowsum);
  else
    k_subln_quant<0><<<grid, block, 0, stream>>>(xv, (int)k, gain, eps_n, xq, scale, rowsum);
  return hipGetLastError();
}

}  // namespace bl
