// Step A0: absmean ternarisation and 2-bit packing of a latent weight matrix.
//
// "BitNet解读" (markgoyens.top), weight quantisation function: the scale is
// the mean |W| over the whole matrix (eq. (3)); weights are divided by
// scale + eps (eq. (1)) and RoundClip'ed to {-1, 0, +1} (eq. (2)).  The
// 2B4T report, section 5.1, stores four ternary values per 8-bit integer.
//
// gamma must be bit-identical however the sum is split over the GPU, so it is
// computed exactly: every |w| is m * 2^(e-150) with a 24-bit integer m and a
// biased exponent e (subnormals use e = 1 without the hidden bit).  The
// integers m are summed per exponent in uint64 (at most 2^26 * 2^10 entries
// of < 2^24 each stay below 2^64), the 254 bucket sums are combined into one
// 384-bit integer, and that is rounded once to binary64, divided by N*K in
// binary64 and rounded to binary32.
#include "bl_internal.h"

namespace bl {
namespace {

constexpr int kHistThreads = 256;
constexpr int kHistWaves = kHistThreads / 64;

__global__ void k_zero_u64(unsigned long long* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

__device__ __forceinline__ void hist_add(unsigned long long* h, float v) {
  const uint32_t u = __float_as_uint(v) & 0x7fffffffu;
  uint32_t e = u >> 23;
  uint32_t m = u & 0x7fffffu;
  if (e) m |= 0x800000u; else e = 1;
  if (m) atomicAdd(&h[e], (unsigned long long)m);
}

// Grid-stride pass over all N*K weights; one LDS histogram per wave cuts
// contention, then each block adds its sums to the global buckets.
__global__ __launch_bounds__(kHistThreads) void k_gamma_hist(const float4* __restrict__ w4,
                                                             int64_t n4,
                                                             unsigned long long* __restrict__ buckets) {
  __shared__ unsigned long long h[kHistWaves][kGammaBuckets];
  for (int i = threadIdx.x; i < kHistWaves * kGammaBuckets; i += kHistThreads)
    (&h[0][0])[i] = 0ull;
  __syncthreads();
  unsigned long long* mine = h[threadIdx.x >> 6];
  const int64_t stride = (int64_t)gridDim.x * kHistThreads;
  for (int64_t i = (int64_t)blockIdx.x * kHistThreads + threadIdx.x; i < n4; i += stride) {
    const float4 v = w4[i];
    hist_add(mine, v.x);
    hist_add(mine, v.y);
    hist_add(mine, v.z);
    hist_add(mine, v.w);
  }
  __syncthreads();
  for (int b = threadIdx.x; b < kGammaBuckets; b += kHistThreads) {
    unsigned long long s = 0;
#pragma unroll
    for (int wv = 0; wv < kHistWaves; ++wv) s += h[wv][b];
    if (s) atomicAdd(&buckets[b], s);
  }
}

// One thread: exact big-integer combine, single rounding to binary64, mean.
__global__ void k_gamma_finalize(const unsigned long long* __restrict__ buckets, int64_t count,
                                 float* __restrict__ gamma) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  constexpr int kLimbs = 12;  // 384 bits > 253 + 64 + 8
  uint32_t limb[kLimbs];
  for (int i = 0; i < kLimbs; ++i) limb[i] = 0;
  for (int b = 1; b < 255; ++b) {
    const unsigned long long v = buckets[b];
    if (!v) continue;
    const int sh = b - 1;          // value = v * 2^(b-1) * 2^-149
    const int l0 = sh >> 5, o = sh & 31;
    const unsigned long long lo = v << o;
    const uint32_t part[3] = {(uint32_t)lo, (uint32_t)(lo >> 32),
                              o ? (uint32_t)(v >> (64 - o)) : 0u};
    unsigned long long carry = 0;
    for (int i = l0; i < kLimbs; ++i) {
      const int pi = i - l0;
      unsigned long long s = (unsigned long long)limb[i] + carry + (pi < 3 ? part[pi] : 0u);
      limb[i] = (uint32_t)s;
      carry = s >> 32;
      if (pi >= 2 && !carry) break;
    }
  }
  int top = -1;
  for (int i = kLimbs - 1; i >= 0 && top < 0; --i)
    if (limb[i]) top = i * 32 + (31 - __builtin_clz(limb[i]));
  double sum;
  if (top < 0) {
    sum = 0.0;
  } else if (top <= 52) {
    const unsigned long long x = ((unsigned long long)limb[1] << 32) | limb[0];
    sum = ldexp((double)x, -149);
  } else {
    auto bit = [&](int i) -> uint32_t { return (limb[i >> 5] >> (i & 31)) & 1u; };
    unsigned long long m = 0;
    for (int i = top; i >= top - 52; --i) m = (m << 1) | bit(i);
    const uint32_t rnd = bit(top - 53);
    uint32_t sticky = 0;
    for (int i = top - 54; i >= 0 && !sticky; --i) sticky |= bit(i);
    int e = top - 52;
    if (rnd && (sticky || (m & 1ull))) {
      ++m;
      if (m == (1ull << 53)) { m >>= 1; ++e; }
    }
    sum = ldexp((double)m, e - 149);
  }
  const double mean = sum / (double)count;
  gamma[0] = (float)mean;
}

__device__ __forceinline__ uint32_t tern_code(float w, float d) {
  const float u = w / d;  // IEEE binary32 division
  const float r = fminf(fmaxf(rintf(u), -1.0f), 1.0f);
  return (uint32_t)((int)r + 1);
}

// One thread per packed word: 16 consecutive weights of a row.
__global__ __launch_bounds__(256) void k_ternarize_pack(const float4* __restrict__ w4,
                                                        int64_t nwords,
                                                        const float* __restrict__ gamma,
                                                        uint32_t* __restrict__ packed) {
  const float d = gamma[0] + kEps;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords; i += stride) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // float4 j holds k = 16g + 4j + {0,1,2,3}
      const float4 v = w4[i * 4 + j];
      word |= tern_code(v.x, d) << (2 * j);
      word |= tern_code(v.y, d) << (8 + 2 * j);
      word |= tern_code(v.z, d) << (16 + 2 * j);
      word |= tern_code(v.w, d) << (24 + 2 * j);
    }
    packed[i] = word;
  }
}

// Row interleave of two packed matrices with the same shape: out row 2i is
// row i of a, out row 2i + 1 row i of b; one packed word per thread step.
__global__ __launch_bounds__(256) void k_interleave(const uint32_t* __restrict__ a,
                                                    const uint32_t* __restrict__ b, int64_t k16,
                                                    int64_t total, uint32_t* __restrict__ out) {
  for (int64_t w = blockIdx.x * 256ll + threadIdx.x; w < total; w += (int64_t)gridDim.x * 256) {
    const int64_t row = w / k16, col = w - row * k16;
    const uint32_t* src = (row & 1) ? b : a;
    out[w] = src[(row >> 1) * k16 + col];
  }
}

int grid_for(int64_t items, int threads, int cap) {
  int64_t g = (items + threads - 1) / threads;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

hipError_t launch_gamma(const float* w, int64_t n, int64_t k, float* gamma,
                        unsigned long long* buckets, hipStream_t stream) {
  const int64_t count = n * k;
  k_zero_u64<<<1, kGammaBuckets, 0, stream>>>(buckets, kGammaBuckets);
  const int64_t n4 = count / 4;
  k_gamma_hist<<<grid_for(n4, kHistThreads, 2048), kHistThreads, 0, stream>>>(
      reinterpret_cast<const float4*>(w), n4, buckets);
  k_gamma_finalize<<<1, 64, 0, stream>>>(buckets, count, gamma);
  return hipGetLastError();
}

hipError_t launch_pack(const float* w, int64_t n, int64_t k, uint8_t* packed, float* gamma,
                       unsigned long long* buckets, hipStream_t stream) {
  const int64_t count = n * k;
  hipError_t e = launch_gamma(w, n, k, gamma, buckets, stream);
  if (e != hipSuccess) return e;
  const int64_t nwords = count / 16;
  k_ternarize_pack<<<grid_for(nwords, 256, 65536), 256, 0, stream>>>(
      reinterpret_cast<const float4*>(w), nwords, gamma, reinterpret_cast<uint32_t*>(packed));
  return hipGetLastError();
}

hipError_t launch_interleave(const uint8_t* a, const uint8_t* b, int64_t n, int64_t k,
                             uint8_t* out, hipStream_t stream) {
  const int64_t k16 = k / 16, total = 2 * n * k16;
  k_interleave<<<grid_for(total, 256, 65536), 256, 0, stream>>>(
      reinterpret_cast<const uint32_t*>(a), reinterpret_cast<const uint32_t*>(b), k16, total,
      reinterpret_cast<uint32_t*>(out));
  return hipGetLastError();
}

}  // namespace bl
