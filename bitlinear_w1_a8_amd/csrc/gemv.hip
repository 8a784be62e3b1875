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
#include "bitlinear.h"
#include "bl_internal.h"

namespace bl {
namespace {

constexpr int kGemvTokens = 64;   // tokens per launch (4 MFMA column tiles)
constexpr int kGemvStage = 8;     // 16-byte activation vectors staged per thread

template <int VEC, int RT, int NTT, int U>
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

  // Each pass: a wave takes U consecutive chunks and issues all their loads
  // before the first MFMA, so U * 1 KiB per row tile is in flight per wave.
  for (int c0 = wave * U; c0 < nchunks; c0 += nwaves * U) {
    uint32_t wv[U][RT][VEC];
    uint32_t xv[U][NTT][4 * VEC];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int wi = (c0 + u) * 4 * VEC + qg * VEC;   // first packed word of this lane
      const bool kvalid = wi < K16;                   // VEC divides K16 when VEC > 1
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        if constexpr (VEC == 4) {
          const uint4 w4 =
              kvalid ? *reinterpret_cast<const uint4*>(wrow[rt] + wi) : make_uint4(0, 0, 0, 0);
          wv[u][rt][0] = w4.x; wv[u][rt][1] = w4.y; wv[u][rt][2] = w4.z; wv[u][rt][3] = w4.w;
        } else {
#pragma unroll
          for (int v = 0; v < VEC; ++v) wv[u][rt][v] = kvalid ? wrow[rt][wi + v] : 0u;
        }
      }
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
        const bool ok = kvalid && tvalid[tt];
        const uint4* src = reinterpret_cast<const uint4*>(xrow[tt] + (int64_t)wi * 16);
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          const uint4 x4 = ok ? src[v] : make_uint4(0, 0, 0, 0);
          xv[u][tt][4 * v + 0] = x4.x; xv[u][tt][4 * v + 1] = x4.y;
          xv[u][tt][4 * v + 2] = x4.z; xv[u][tt][4 * v + 3] = x4.w;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int d = 0; d < 4 * VEC; ++d)
          qs[tt] = __builtin_amdgcn_sdot4((int)xv[u][tt][d], 0x01010101, qs[tt], false);
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const uint32_t w = wv[u][rt][v];
          const v4i a = {(int)codes_of(w, 0), (int)codes_of(w, 1), (int)codes_of(w, 2),
                         (int)codes_of(w, 3)};
#pragma unroll
          for (int tt = 0; tt < NTT; ++tt) {
            const v4i b = {(int)xv[u][tt][4 * v + 0], (int)xv[u][tt][4 * v + 1],
                           (int)xv[u][tt][4 * v + 2], (int)xv[u][tt][4 * v + 3]};
            acc[rt][tt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[rt][tt], 0, 0, 0);
          }
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

// Software-pipelined variant for T <= 16 and K % 256 == 0 (the decode case).
//
// Per chunk (256 k of a 16-row tile) a lane holds four packed words w_v.
// Instead of shifting every 2-bit field down, three of the four fields are
// only masked: w & 0x03030303, w & 0x0C0C0C0C and w & 0x30303030 hold c,
// 4c and 16c in each byte (all still non-negative int8), and only the top
// field needs a shift.  Slice j of the four words forms one MFMA operand, and
// each scale accumulates separately; the exact sums are divided by 4 and 16
// once at the end (they are exact multiples).  The activation bytes are laid
// out in LDS so that the matching B operand of slice j is one 16-byte read:
// within every 64-byte group the 4x4 dword matrix (word v, slice j) is
// stored transposed.  The token's sum of q over K, which removes the code
// offset (c = t + 1), is taken once per block.
//
// Each wave walks its chunks with P loads in flight: the load of chunk i+P
// is issued as soon as chunk i is consumed.
//
// One launch serves a group of independent problems (blocks are dealt out
// problem by problem).  MODE selects the activation input: kInt8 reads the
// int8 activations and absmax of a separate act-quant step; kBf16 / kF32
// read raw activations and quantise them in the block (step A1 fused): every
// block derives the token absmax itself, scales, rounds half to even and
// clips exactly as the act-quant kernel does, and the problem's first block
// also stores the int8 activations and absmax.
enum PipeMode { kInt8 = 0, kBf16 = 1, kF32 = 2 };

struct PipeProblem {
  const uint32_t* packed;
  const float* gamma;
  const void* x;          // int8 activations (kInt8) or raw bf16 / f32
  const float* absmax;    // kInt8: per-token absmax from act-quant
  float* y;
  int32_t* acc;           // optional exact sums
  int8_t* xq_out;         // fused modes: quantised activations out (first block)
  float* absmax_out;      // fused modes: absmax out (first block)
  int N, K, block0;
};
constexpr int kMaxGroup = 8;
struct PipeGroup {
  PipeProblem p[kMaxGroup];
  int count, T;
};

// DPP row reductions (16 lanes), then the four rows through readlane.
__device__ __forceinline__ int wave_max_nonneg(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false));  // row_mirror
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ int wave_sum_i(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
         __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

// element e of a raw 16-byte activation vector, widened exactly to binary32
template <int MODE>
__device__ __forceinline__ float raw_elem(const uint4& v, int e) {
  if constexpr (MODE == kBf16) {
    const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  } else {
    return __uint_as_float(e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w);
  }
}

template <int P, int MODE>
__global__ __launch_bounds__(1024) void k_gemv_pipe(const PipeGroup grp) {
  extern __shared__ __align__(16) unsigned char smem[];
  int pi = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i)
    if (i < grp.count && (int)blockIdx.x >= grp.p[i].block0) pi = i;
  const PipeProblem& pr = grp.p[pi];
  const int T = grp.T, N = pr.N, K = pr.K;

  const int lane = threadIdx.x & 63, nwaves = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qg = lane >> 4, r = lane & 15;
  const int K16 = K >> 4;
  const int nchunks = K16 >> 4;                     // 16 words (256 k) per chunk
  const int n0 = ((int)blockIdx.x - pr.block0) * 16;
  // LDS: [256 B zeros][T x (K + 16) activation bytes, transposed per 64 B]
  //      [16 row sums][16 absmax bits][partials].  The 16-byte pad per token
  //      spreads the tokens of one B-operand read over different banks.
  const int xs = (K >> 2) + 4;                      // token stride in dwords
  uint32_t* zero = reinterpret_cast<uint32_t*>(smem);
  uint32_t* xl = zero + 64;
  int* rsum = reinterpret_cast<int*>(xl + T * xs);
  int* amax = rsum + 16;
  int* red = amax + 16;

  int n = n0 + r;
  n = n < N ? n : N - 1;
  const uint4* wrow = reinterpret_cast<const uint4*>(pr.packed + (int64_t)n * K16) + qg;
  const int my = (nchunks - wave + nwaves - 1) / nwaves;   // chunks of this wave (>= 1)
  auto chunk_of = [&](int i) { return wave + (i < my ? i : my - 1) * nwaves; };

  // Issue order matters: vector loads retire in order, so anything waited on
  // before the main loop (the activations) is issued before the weight
  // prefetch, which then stays in flight through the staging and the barrier.
  constexpr int kStage = kGemvStage;
  constexpr int E = MODE == kInt8 ? 16 : MODE == kBf16 ? 8 : 4;  // elements per 16 bytes
  const int per_tok = K / E, nvec = T * per_tok;
  const uint4* src = reinterpret_cast<const uint4*>(pr.x);
  uint4 sv[kStage];
#pragma unroll
  for (int m = 0; m < kStage; ++m) {
    const int i = threadIdx.x + m * blockDim.x;
    sv[m] = src[i < nvec ? i : nvec - 1];
  }
  // the epilogue's scalars, fetched early so their latency hides under the loop
  const float g = pr.gamma[0];
  float am = 0.0f;
  if constexpr (MODE == kInt8) am = pr.absmax[threadIdx.x < 16 * T ? (threadIdx.x >> 4) : 0];

  uint4 buf[P];
#pragma unroll
  for (int j = 0; j < P; ++j) buf[j] = wrow[(size_t)chunk_of(j) * 4];

  if (threadIdx.x < 64) zero[threadIdx.x] = 0u;
  if (threadIdx.x < 32) rsum[threadIdx.x] = 0;      // row sums and absmax bits
  // 16 int8 activations = word v = iv & 3 of a 64-byte group; dword (v, j)
  // of the group is stored at position (j, v).
  auto xq_dword = [&](int t, int iv, int j) -> uint32_t* {
    return xl + t * xs + (iv >> 2) * 16 + (iv & 3) + 4 * j;
  };
  if constexpr (MODE == kInt8) {
#pragma unroll
    for (int m = 0; m < kStage; ++m) {
      const int i = threadIdx.x + m * blockDim.x;
      if (i < nvec) {
        const int t = i / per_tok, iv = i - t * per_tok;
        *xq_dword(t, iv, 0) = sv[m].x; *xq_dword(t, iv, 1) = sv[m].y;
        *xq_dword(t, iv, 2) = sv[m].z; *xq_dword(t, iv, 3) = sv[m].w;
      }
    }
    // (the host guarantees nvec <= kStage * blockDim: one round covers it)
  } else {
    // Step A1 in the block: absmax per token (T <= 4) ...
    int tmax[4] = {0, 0, 0, 0};
#pragma unroll
    for (int m = 0; m < kStage; ++m) {
      const int i = threadIdx.x + m * blockDim.x;
      if (i < nvec) {
        const int t = i / per_tok;
        int mx = 0;
#pragma unroll
        for (int e = 0; e < E; ++e)
          mx = max(mx, (int)(__float_as_uint(raw_elem<MODE>(sv[m], e)) & 0x7fffffffu));
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
          if (t == tt) tmax[tt] = max(tmax[tt], mx);
      }
    }
    __syncthreads();                                // amax cleared
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      if (tt < T) {
        const int wm = wave_max_nonneg(tmax[tt]);   // non-negative bit patterns order as values
        if (lane == 0) atomicMax(&amax[tt], wm);
      }
    }
    __syncthreads();
    // ... then scale, round half to even, clip, and lay out as int8
    float sc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
      sc[tt] = tt < T ? kQb / fmaxf(__uint_as_float((uint32_t)amax[tt]), kEps) : 0.0f;
    int tsum[4] = {0, 0, 0, 0};
    const bool first = n0 == 0;
#pragma unroll
    for (int m = 0; m < kStage; ++m) {
      const int i = threadIdx.x + m * blockDim.x;
      if (i < nvec) {
        const int t = i / per_tok, ie = i - t * per_tok;   // vector index within the token
        float s = sc[0];
#pragma unroll
        for (int tt = 1; tt < 4; ++tt)
          if (t == tt) s = sc[tt];
        uint32_t d[E / 4];
        int part = 0;
#pragma unroll
        for (int w = 0; w < E / 4; ++w) {
          uint32_t word = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const float v = raw_elem<MODE>(sv[m], 4 * w + b) * s;   // one binary32 product
            const int q = (int)fminf(fmaxf(rintf(v), -kQb), kQb);
            part += q;
            word |= (uint32_t)(q & 0xff) << (8 * b);
          }
          d[w] = word;
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
          if (t == tt) tsum[tt] += part;
        // E elements start at k = ie * E: int8 vector iv, first dword j0
        const int k0 = ie * E, iv = k0 >> 4, j0 = (k0 & 15) >> 2;
#pragma unroll
        for (int w = 0; w < E / 4; ++w) *xq_dword(t, iv, j0 + w) = d[w];
        if (first && pr.xq_out) {
          int8_t* dst = pr.xq_out + (int64_t)t * K + k0;
          if constexpr (E == 8)
            *reinterpret_cast<uint2*>(dst) = make_uint2(d[0], d[E / 4 - 1]);
          else
            *reinterpret_cast<uint32_t*>(dst) = d[0];
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      if (tt < T) {
        const int ws = wave_sum_i(tsum[tt]);
        if (lane == 0) atomicAdd(&rsum[tt], ws);
      }
    }
    if (first && pr.absmax_out && threadIdx.x < T)
      pr.absmax_out[threadIdx.x] = __uint_as_float((uint32_t)amax[threadIdx.x]);
  }
  __syncthreads();

  // B operand address: lanes of tokens past T read the zero block (stride 0)
  const uint4* xb = reinterpret_cast<const uint4*>(r < T ? xl + r * xs + qg * 16 : zero);
  const int xstride = r < T ? 16 : 0;              // uint4 per chunk

  v4i a1 = {0, 0, 0, 0}, a4 = {0, 0, 0, 0}, a16 = {0, 0, 0, 0};
  struct Slices { v4i s0, s1, s2, s3; };
  auto unpack = [](const uint4& w4) {
    Slices q;
    q.s0 = v4i{(int)(w4.x & 0x03030303u), (int)(w4.y & 0x03030303u),
               (int)(w4.z & 0x03030303u), (int)(w4.w & 0x03030303u)};
    q.s1 = v4i{(int)(w4.x & 0x0C0C0C0Cu), (int)(w4.y & 0x0C0C0C0Cu),
               (int)(w4.z & 0x0C0C0C0Cu), (int)(w4.w & 0x0C0C0C0Cu)};
    q.s2 = v4i{(int)(w4.x & 0x30303030u), (int)(w4.y & 0x30303030u),
               (int)(w4.z & 0x30303030u), (int)(w4.w & 0x30303030u)};
    q.s3 = v4i{(int)((w4.x >> 6) & 0x03030303u), (int)((w4.y >> 6) & 0x03030303u),
               (int)((w4.z >> 6) & 0x03030303u), (int)((w4.w >> 6) & 0x03030303u)};
    return q;
  };
  auto mma = [&](const Slices& q, int c) {
    const uint4* xc = xb + c * xstride;
    const uint4 b0 = xc[0], b1 = xc[1], b2 = xc[2], b3 = xc[3];
    a1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(
        q.s0, v4i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w}, a1, 0, 0, 0);
    a4 = __builtin_amdgcn_mfma_i32_16x16x64_i8(
        q.s1, v4i{(int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w}, a4, 0, 0, 0);
    a16 = __builtin_amdgcn_mfma_i32_16x16x64_i8(
        q.s2, v4i{(int)b2.x, (int)b2.y, (int)b2.z, (int)b2.w}, a16, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(
        q.s3, v4i{(int)b3.x, (int)b3.y, (int)b3.z, (int)b3.w}, a1, 0, 0, 0);
  };

  int i0 = 0;
  for (; i0 + P <= my; i0 += P) {
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int i = i0 + j;
      // consume buf[j] first, then refill the same registers: no copies, and
      // the wait before the masks is only for this one load (P-1 stay in flight)
      const Slices q = unpack(buf[j]);
      buf[j] = wrow[(size_t)chunk_of(i + P) * 4];
      __builtin_amdgcn_sched_barrier(0);
      mma(q, wave + i * nwaves);
    }
  }
#pragma unroll
  for (int j = 0; j < P; ++j)   // the last my % P chunks are already in buf[0..]
    if (i0 + j < my) mma(unpack(buf[j]), wave + (i0 + j) * nwaves);

#pragma unroll
  for (int v = 0; v < 4; ++v)
    red[(wave * 4 + v) * 64 + lane] = a1[v] + (a4[v] >> 2) + (a16[v] >> 4);

  if constexpr (MODE == kInt8) {
    // sum of q per token (removes the code offset), read back from LDS
    for (int t = 0; t < T; ++t) {
      const uint4* xt = reinterpret_cast<const uint4*>(xl + t * xs);
      int part = 0;
      for (int i = threadIdx.x; i < (K >> 4); i += blockDim.x) {
        const uint4 v = xt[i];
        part = __builtin_amdgcn_sdot4((int)v.x, 0x01010101, part, false);
        part = __builtin_amdgcn_sdot4((int)v.y, 0x01010101, part, false);
        part = __builtin_amdgcn_sdot4((int)v.z, 0x01010101, part, false);
        part = __builtin_amdgcn_sdot4((int)v.w, 0x01010101, part, false);
      }
      part = wave_sum_i(part);
      if (lane == 0) atomicAdd(&rsum[t], part);
    }
  }
  __syncthreads();
  // 16 * T <= 256 outputs and blockDim >= 64: thread idx < 16 * T owns one
  for (int idx = threadIdx.x; idx < 16 * T; idx += blockDim.x) {
    const int i = idx & 15, tl = idx >> 4;
    const int nn = n0 + i;
    if (nn >= N) continue;
    const int slot = i & 3, ln = (i >> 2) * 16 + tl;
    int sum = -rsum[tl];
    for (int wv = 0; wv < nwaves; ++wv) sum += red[(wv * 4 + slot) * 64 + ln];
    const int64_t o = (int64_t)tl * N + nn;
    if (pr.acc) pr.acc[o] = sum;
    float a_t;
    if constexpr (MODE == kInt8) a_t = idx == (int)threadIdx.x ? am : pr.absmax[tl];
    else a_t = __uint_as_float((uint32_t)amax[tl]);
    pr.y[o] = (float)sum * out_scale(g, a_t);
  }
}

// Launch-shape tunables (compile-time so variants can be built and compared).
#ifndef BL_GEMV_U
#define BL_GEMV_U 4          // chunks whose loads a wave issues together
#endif
#ifndef BL_GEMV_MAXW
#define BL_GEMV_MAXW 8       // most waves per block (they split K)
#endif

template <int VEC, int RT, int NTT, int U>
void run(const uint8_t* packed, const float* gamma, const int8_t* xq, const float* absmax,
         int t, int n, int k, float* y, int32_t* acc, hipStream_t stream) {
  const int k16 = k / 16;
  const int nchunks = (k16 + 4 * VEC - 1) / (4 * VEC);
  int nw = (nchunks + U - 1) / U;       // one pass of U chunks per wave where possible
  if (nw < 1) nw = 1;
  if (nw > BL_GEMV_MAXW) nw = BL_GEMV_MAXW;
  const int grid = (n + 16 * RT - 1) / (16 * RT);
  const size_t lds = (size_t)nw * RT * NTT * 4 * 64 * sizeof(int);
  k_gemv<VEC, RT, NTT, U><<<grid, nw * 64, lds, stream>>>(
      reinterpret_cast<const uint32_t*>(packed), gamma, xq, absmax, t, n, k, y, acc);
}

template <int VEC>
void run_tokens(const uint8_t* packed, const float* gamma, const int8_t* xq,
                const float* absmax, int t, int n, int k, float* y, int32_t* acc,
                hipStream_t stream) {
  if (t <= 16)
    run<VEC, 1, 1, BL_GEMV_U>(packed, gamma, xq, absmax, t, n, k, y, acc, stream);
  else if (t <= 32)
    run<VEC, 2, 2, (BL_GEMV_U > 2 ? 2 : BL_GEMV_U)>(packed, gamma, xq, absmax, t, n, k, y, acc,
                                                    stream);
  else
    run<VEC, 2, 4, 1>(packed, gamma, xq, absmax, t, n, k, y, acc, stream);
}

}  // namespace

#ifndef BL_GEMV_PIPE_P
#define BL_GEMV_PIPE_P 6          // chunks in flight per wave in the pipelined kernel
#endif
#ifndef BL_GEMV_PIPE_WAVES
#define BL_GEMV_PIPE_WAVES 2048   // total waves aimed for (about 8 per CU)
#endif
#ifndef BL_GEMV_PIPE_MINCPW
#define BL_GEMV_PIPE_MINCPW 4     // fewest chunks per wave when splitting K
#endif
#ifndef BL_GEMV_PIPE_XLDS
#define BL_GEMV_PIPE_XLDS 32768  // largest T*K staged in LDS
#endif

// Waves per block of the pipelined kernel.  Large grids do best with few,
// long-running waves (each streams many chunks); small grids need K split over
// more waves to have enough loads in flight.  Aim for about
// BL_GEMV_PIPE_WAVES waves in total with at least BL_GEMV_PIPE_MINCPW chunks
// each, and enough threads to stage the activations in one round
// (elems_per_vec elements per 16-byte vector).
int pipe_waves(int64_t t, int64_t blocks, int64_t k, int elems_per_vec) {
  const int nchunks = (int)(k / 256);
  int nw = (int)((BL_GEMV_PIPE_WAVES + blocks - 1) / blocks);
  int cap = nchunks / BL_GEMV_PIPE_MINCPW;
  if (cap < 1) cap = 1;
  if (nw > cap) nw = cap;
  const int64_t vecs = t * k / elems_per_vec;
  const int need = (int)((vecs + 64 * kGemvStage - 1) / (64 * kGemvStage));
  if (nw < need) nw = need;
  if (nw > nchunks) nw = nchunks;
  return nw;
}

bool pipe_shape_ok(int64_t t, int64_t k, int elems_per_vec, int max_t) {
  if (!(t <= max_t && (k % 256) == 0 && t * k <= BL_GEMV_PIPE_XLDS)) return false;
  const int nw = pipe_waves(t, 1, k, elems_per_vec);  // the fewest-waves case bounds staging
  return nw <= 16 && t * k / elems_per_vec <= (int64_t)16 * 64 * kGemvStage;
}

bool pipe_ok(int64_t t, int64_t n, int64_t k, const void* packed, const void* xq) {
  (void)n;
  return pipe_shape_ok(t, k, 16, 16) && (reinterpret_cast<uintptr_t>(packed) % 16) == 0 &&
         (reinterpret_cast<uintptr_t>(xq) % 16) == 0;
}

size_t pipe_lds(int64_t t, int64_t k, int nw) {
  return 256 + (size_t)t * (k + 16) + 32 * sizeof(int) + (size_t)nw * 4 * 64 * sizeof(int);
}

template <int MODE>
hipError_t run_pipe_group(const PipeGroup& grp, int blocks, int nw, size_t lds,
                          hipStream_t stream) {
  k_gemv_pipe<BL_GEMV_PIPE_P, MODE><<<blocks, nw * 64, lds, stream>>>(grp);
  return hipGetLastError();
}

void run_pipe(const uint8_t* packed, const float* gamma, const int8_t* xq, const float* absmax,
              int t, int n, int k, float* y, int32_t* acc, hipStream_t stream) {
  PipeGroup grp = {};
  grp.count = 1;
  grp.T = t;
  grp.p[0] = PipeProblem{reinterpret_cast<const uint32_t*>(packed), gamma, xq, absmax, y, acc,
                         nullptr, nullptr, n, k, 0};
  const int blocks = (n + 15) / 16;
  int nw = pipe_waves(t, blocks, k, 16);
  if (nw * 64 * kGemvStage < (int64_t)t * k / 16) nw = (int)((t * k / 16 + 64 * kGemvStage - 1) / (64 * kGemvStage));
  run_pipe_group<kInt8>(grp, blocks, nw, pipe_lds(t, k, nw), stream);
}

hipError_t launch_linear_group(const bl_linear* probs, int count, int64_t t, int bf16,
                               hipStream_t stream) {
  const int E = bf16 ? 8 : 4;
  bool fused = count <= kMaxGroup;
  for (int i = 0; fused && i < count; ++i) {
    fused = pipe_shape_ok(t, probs[i].K, E, 4) &&
            (reinterpret_cast<uintptr_t>(probs[i].x) % 16) == 0 &&
            (reinterpret_cast<uintptr_t>(probs[i].packed) % 16) == 0;
  }
  if (!fused) {  // act-quant then forward, problem by problem
    for (int i = 0; i < count; ++i) {
      const bl_linear& q = probs[i];
      hipError_t e = launch_quant(q.x, bf16, t, q.K, q.xq, q.absmax, nullptr, stream);
      if (e != hipSuccess) return e;
      e = launch_gemv(q.packed, q.gamma, q.xq, q.absmax, t, q.N, q.K, q.y, q.acc, stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  PipeGroup grp = {};
  grp.count = count;
  grp.T = (int)t;
  int blocks = 0;
  int64_t kmax = 0;
  for (int i = 0; i < count; ++i) {
    const bl_linear& q = probs[i];
    grp.p[i] = PipeProblem{reinterpret_cast<const uint32_t*>(q.packed), q.gamma, q.x, nullptr,
                           q.y, q.acc, q.xq, q.absmax, (int)q.N, (int)q.K, blocks};
    blocks += (int)((q.N + 15) / 16);
    if (q.K > kmax) kmax = q.K;
  }
  // one block shape for the group: waves for the widest K, staging for every K
  int nw = pipe_waves(t, blocks, kmax, E);
  for (int i = 0; i < count; ++i) {
    const int need = (int)((t * probs[i].K / E + 64 * kGemvStage - 1) / (64 * kGemvStage));
    if (nw < need) nw = need;
  }
  if (nw > 16) nw = 16;
  const size_t lds = pipe_lds(t, kmax, nw);
  return bf16 ? run_pipe_group<kBf16>(grp, blocks, nw, lds, stream)
              : run_pipe_group<kF32>(grp, blocks, nw, lds, stream);
}

hipError_t launch_gemv(const uint8_t* packed, const float* gamma, const int8_t* xq,
                       const float* absmax, int64_t t, int64_t n, int64_t k, float* y,
                       int32_t* acc, hipStream_t stream) {
  if (pipe_ok(t, n, k, packed, xq)) {
    run_pipe(packed, gamma, xq, absmax, (int)t, (int)n, (int)k, y, acc, stream);
    return hipGetLastError();
  }
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
