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
#include <mutex>

#include "bl_internal.h"

namespace bl {

// Device-resident buckets of bitlinear_pack_weights_noalloc, for callers that
// cannot allocate: one copy per device, held until the process ends.  In host
// code this name is only a stand-in for the symbol; the device address comes
// from hipGetSymbolAddress (scratch_buckets below) and is the only form ever
// passed to a kernel or a copy.
static __device__ __align__(256) unsigned long long scratch[kGammaBuckets];

namespace {

constexpr int kHistThreads = 256;
constexpr int kHistWaves = kHistThreads / 64;
#ifndef BL_GAMMA_HIST_VPT
#define BL_GAMMA_HIST_VPT 16            // 16-byte vectors per thread the histogram grid aims for
#endif

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

// Grid-stride pass over all N*K weights, four 16-byte loads in flight per
// thread; one LDS histogram per wave cuts contention, then each block adds
// its sums to the global buckets.
__global__ __launch_bounds__(kHistThreads) void k_gamma_hist(const float4* __restrict__ w4,
                                                             int64_t n4,
                                                             unsigned long long* __restrict__ buckets) {
  __shared__ unsigned long long h[kHistWaves][kGammaBuckets];
  for (int i = threadIdx.x; i < kHistWaves * kGammaBuckets; i += kHistThreads)
    (&h[0][0])[i] = 0ull;
  __syncthreads();
  unsigned long long* mine = h[threadIdx.x >> 6];
  const int64_t stride = (int64_t)gridDim.x * kHistThreads;
  int64_t i = (int64_t)blockIdx.x * kHistThreads + threadIdx.x;
  for (; i + 3 * stride < n4; i += 4 * stride) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = w4[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      hist_add(mine, v[u].x);
      hist_add(mine, v[u].y);
      hist_add(mine, v[u].z);
      hist_add(mine, v[u].w);
    }
  }
  for (; i < n4; i += stride) {
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

// One wave: the exact sum of v_b * 2^(b - 1) over buckets b = 1 .. 254 (units
// of 2^-149) as a 384-bit integer, rounded once to binary64; then the mean.
// Lane l takes buckets 4l .. 4l + 3, whose pieces (each v_b << ((b - 1) % 32),
// 96 bits) fall in four consecutive 32-bit words from word (4l - 1) / 32, and
// adds them into twelve 64-bit word sums in LDS (below 64 lanes x 4 pieces of
// 32 bits each, so none overflows); one lane then propagates the carries.
__global__ __launch_bounds__(64) void k_gamma_finalize(const unsigned long long* __restrict__ buckets,
                                                       int64_t count, float* __restrict__ gamma) {
  constexpr int kLimbs = 12;  // 384 bits > 253 + 64 + 8
  __shared__ unsigned long long wsum[kLimbs];
  __shared__ uint32_t limb[kLimbs];
  const int l = threadIdx.x;
  if (l < kLimbs) wsum[l] = 0ull;
  __syncthreads();
  const int w0 = max(4 * l - 1, 0) >> 5;
  unsigned long long win[4] = {0ull, 0ull, 0ull, 0ull};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int b = 4 * l + j;
    const unsigned long long v = (b >= 1 && b <= 254) ? buckets[b] : 0ull;
    const int off = max(b - 1, 0), sh = off & 31;
    const unsigned long long lo = v << sh;
    const uint32_t p0 = (uint32_t)lo, p1 = (uint32_t)(lo >> 32);
    const uint32_t p2 = sh ? (uint32_t)(v >> (64 - sh)) : 0u;
    const bool d0 = (off >> 5) == w0;   // else one word further up
    win[0] += d0 ? p0 : 0u;
    win[1] += d0 ? p1 : p0;
    win[2] += d0 ? p2 : p1;
    win[3] += d0 ? 0u : p2;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (win[i]) atomicAdd(&wsum[w0 + i], win[i]);
  __syncthreads();
  if (l == 0) {
    unsigned long long carry = 0;
    for (int i = 0; i < kLimbs; ++i) {
      const unsigned long long s = wsum[i] + carry;   // < 2^41 + 2^10
      limb[i] = (uint32_t)s;
      carry = s >> 32;
    }
    const double sum = limbs_to_f64(limb, -149);
    const double mean = sum / (double)count;
    gamma[0] = (float)mean;
  }
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

// Blocks of the histogram pass: about BL_GAMMA_HIST_VPT vectors per thread,
// from 256 to 2048 blocks (every block ends with global atomics on the same
// few buckets, so small matrices take fewer blocks).
int hist_grid(int64_t n4) {
  int64_t g = (n4 + (int64_t)kHistThreads * BL_GAMMA_HIST_VPT - 1) /
              ((int64_t)kHistThreads * BL_GAMMA_HIST_VPT);
  const int64_t lo = (n4 + kHistThreads - 1) / kHistThreads;   // one vector per thread
  if (g < 256) g = lo < 256 ? lo : 256;
  if (g > 2048) g = 2048;
  return (int)g;
}

}  // namespace

hipError_t launch_gamma(const float* w, int64_t n, int64_t k, float* gamma,
                        unsigned long long* buckets, hipStream_t stream) {
  const int64_t count = n * k;
  k_zero_u64<<<1, kGammaBuckets, 0, stream>>>(buckets, kGammaBuckets);
  const int64_t n4 = count / 4;
  k_gamma_hist<<<hist_grid(n4), kHistThreads, 0, stream>>>(
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

hipError_t scratch_buckets(hipStream_t stream, unsigned long long** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int cur = 0, dev = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  dev = cur;
  if (stream) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    // Looked up once per device, with that device current.
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = static_cast<unsigned long long*>(addr[dev]);
  return hipSuccess;
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
