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
// total is gathered in 256 uint64 buckets, bucket b counting units of
// 2^(b - 150): most weights through exact fixed-point sums per wave placed
// there as 32-bit pieces, the rest one m at a time (below 2^62 + 2^45 per
// bucket for N*K <= 2^38); the 254 bucket sums are combined into one 384-bit
// integer, and that is rounded once to binary64, divided by N*K in binary64
// and rounded to binary32.
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
#ifndef BL_GAMMA_HIST_VPT
#define BL_GAMMA_HIST_VPT 16            // 16-byte vectors per thread the histogram grid aims for
#endif

__global__ void k_zero_u64(unsigned long long* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

// |w| = m * 2^(e - 150): 24-bit significand, biased exponent (1 for subnormals).
__device__ __forceinline__ void split_abs(float v, uint32_t& m, int& e) {
  const uint32_t u = __float_as_uint(v) & 0x7fffffffu;
  e = (int)(u >> 23);
  m = u & 0x7fffffu;
  if (e) m |= 0x800000u; else e = 1;
}

// The wave's fixed-point sums (lo, hi: integers in units of 2^(u - 150)),
// added over the wave, into the block's buckets: bucket b counts units of
// 2^(b - 150), so 32-bit piece j goes to bucket u + 32j.  A lane's sum is below
// 2^83 (at most 2^19 terms below 2^64), the wave's below 2^89: three pieces.
// Called by every lane of the wave.
__device__ __forceinline__ void flush_fixed(unsigned long long lo, unsigned long long hi, int u,
                                            unsigned long long* h, int lane) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const unsigned long long l2 = __shfl_xor(lo, o), h2 = __shfl_xor(hi, o);
    const unsigned long long s = lo + l2;
    hi += h2 + (s < l2 ? 1ull : 0ull);
    lo = s;
  }
  if (lane == 0) {
    if (lo & 0xffffffffull) atomicAdd(&h[u], lo & 0xffffffffull);
    if (lo >> 32) atomicAdd(&h[u + 32], lo >> 32);
    if (hi) atomicAdd(&h[u + 64], hi);
  }
}

// One wave: the exact sum of v_b * 2^(b - 1) over buckets b = 1 .. 254 (units
// of 2^-149) as a 384-bit integer, rounded once to binary64; then the mean.
// Lane l takes buckets 4l .. 4l + 3, whose pieces (each v_b << ((b - 1) % 32),
// 96 bits) fall in four consecutive 32-bit words from word (4l - 1) / 32, and
// adds them into twelve 64-bit word sums in LDS (below 64 lanes x 4 pieces of
// 32 bits each, so none overflows); one lane then propagates the carries.
constexpr int kGammaLimbs = 12;  // 384 bits > 253 + 64 + 8
__device__ void gamma_finalize_wave(const unsigned long long* buckets, int64_t count,
                                    float* gamma, unsigned long long* wsum, uint32_t* limb_arr,
                                    int l) {
  if (l < kGammaLimbs) wsum[l] = 0ull;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  const int w0 = max(4 * l - 1, 0) >> 5;
  unsigned long long win[4] = {0ull, 0ull, 0ull, 0ull};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int b = 4 * l + j;
    const unsigned long long v =
        (b >= 1 && b <= 254)
            ? __hip_atomic_load(&buckets[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
            : 0ull;
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
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  if (l == 0) {
    uint32_t (&limb)[kGammaLimbs] = *reinterpret_cast<uint32_t(*)[kGammaLimbs]>(limb_arr);
    unsigned long long carry = 0;
    for (int i = 0; i < kGammaLimbs; ++i) {
      const unsigned long long s = wsum[i] + carry;   // < 2^41 + 2^10
      limb[i] = (uint32_t)s;
      carry = s >> 32;
    }
    const double sum = limbs_to_f64(limb, -149);
    const double mean = sum / (double)count;
    gamma[0] = (float)mean;
  }
}

// Grid-stride pass over all N*K weights, four 16-byte loads per lane and
// step, the next step's loads issued before the current step's arithmetic.
// Each wave takes a reference exponent R two binades above the largest of its
// first 16 x 64 weights and every lane adds m << (e - u), u = R - kFixWindow
// (at least 1), for each normal weight with u <= e <= R into a 128-bit
// integer: every term is below 2^64 and the sum is exact.  Other nonzero
// weights (subnormals, or outside that window: none or few in a weight
// matrix) go straight into the block's LDS buckets, and at the end each wave
// adds its lanes' sums and moves the total there as three 32-bit pieces.
// Each block then adds its nonzero buckets to the global ones.
constexpr int kFixWindow = 40;
constexpr int kFixMaxE = 200;   // u + 64 <= 224 stays inside the buckets
__global__ __launch_bounds__(kHistThreads) void k_gamma_hist(const float4* __restrict__ w4,
                                                             int64_t n4,
                                                             unsigned long long* __restrict__ buckets) {
  __shared__ unsigned long long h[kGammaBuckets];
  for (int i = threadIdx.x; i < kGammaBuckets; i += kHistThreads) h[i] = 0ull;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t stride = (int64_t)gridDim.x * kHistThreads;
  // four vectors from i on, stride apart; past the end: zeros (the address
  // clamped, so every load stays in bounds and needs no branch)
  auto load = [&](int64_t i, uint32_t (&b)[16]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t idx = i + q * stride;
      const float4 v = w4[idx < n4 ? idx : n4 - 1];
      const bool in = idx < n4;
      b[4 * q] = in ? __float_as_uint(v.x) : 0u;
      b[4 * q + 1] = in ? __float_as_uint(v.y) : 0u;
      b[4 * q + 2] = in ? __float_as_uint(v.z) : 0u;
      b[4 * q + 3] = in ? __float_as_uint(v.w) : 0u;
    }
  };
  int64_t i = (int64_t)blockIdx.x * kHistThreads + threadIdx.x;
  uint32_t cur[16], nxt[16];
  load(i, cur);                                  // zeros for lanes past the end
  int em = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) em = max(em, (int)((cur[q] & 0x7fffffffu) >> 23));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) em = max(em, __shfl_xor(em, o));
  const int R = min(em + 2, kFixMaxE);           // wave-uniform
  const int u = max(R - kFixWindow, 1);
  const uint32_t span = (uint32_t)(R - u);
  unsigned long long lo = 0ull, hi = 0ull;
  if (i < n4) {
    for (;;) {
      const int64_t in = i + 4 * stride;
      const bool more = in < n4;
      if (more) load(in, nxt);
      uint32_t rare = 0u;                        // nonzero: some weight outside the window
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const uint32_t b = cur[q] & 0x7fffffffu;
        const int d = (int)(b >> 23) - u;        // subnormals and zeros: below the window
        const bool fix = (uint32_t)d <= span;
        const uint32_t m = fix ? ((b & 0x7fffffu) | 0x800000u) : 0u;
        const unsigned long long t = (unsigned long long)m << (d & 63);
        const unsigned long long s = lo + t;
        hi += s < t ? 1ull : 0ull;
        lo = s;
        rare |= fix ? 0u : b;
      }
      if (rare) {                                // rare: outside the window
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          uint32_t m;
          int e;
          split_abs(__uint_as_float(cur[q]), m, e);
          if (m != 0u && (e < u || e > R || (cur[q] & 0x7f800000u) == 0u))
            atomicAdd(&h[e], (unsigned long long)m);
        }
      }
      if (!more) break;
      i = in;
      for (int q = 0; q < 16; ++q) cur[q] = nxt[q];
    }
  }
  flush_fixed(lo, hi, u, h, lane);               // every lane of the wave
  __syncthreads();
  for (int b = threadIdx.x; b < kGammaBuckets; b += kHistThreads) {
    const unsigned long long s = h[b];
    if (s) atomicAdd(&buckets[b], s);
  }
}

__global__ __launch_bounds__(64) void k_gamma_finalize(const unsigned long long* __restrict__ buckets,
                                                       int64_t count, float* __restrict__ gamma) {
  __shared__ unsigned long long wsum[kGammaLimbs];
  __shared__ uint32_t limb[kGammaLimbs];
  gamma_finalize_wave(buckets, count, gamma, wsum, limb, threadIdx.x);
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
