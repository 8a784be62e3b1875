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
#include <atomic>
#include <type_traits>

#include "bitlinear.h"
#include "bl_internal.h"

namespace bl {
namespace {

constexpr int kGemvTokens = 64;   // tokens per launch (4 MFMA column tiles)

template <int VEC, int RT, int NTT, int U>
__global__ __launch_bounds__(512) void k_gemv(const uint32_t* __restrict__ packed,
                                              const float* __restrict__ gamma,
                                              const int8_t* __restrict__ xq,
                                              const float* __restrict__ absmax, int T, int N,
                                              int K, float* __restrict__ y,
                                              int32_t* __restrict__ acc_out,
                                              const float* __restrict__ gamma2,
                                              uint16_t* __restrict__ h,
                                              const int32_t* __restrict__ rowsum) {
  extern __shared__ int red[];  // [nwaves][RT*NTT*4][64]
  const bool derive = rowsum == nullptr;   // sum q here, or take each token's total
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
      if (derive) {
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
          for (int d = 0; d < 4 * VEC; ++d)
            qs[tt] = __builtin_amdgcn_sdot4((int)xv[u][tt][d], 0x01010101, qs[tt], false);
      }
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

  // sum of q over this wave's k for the token of column r: add the 4 lane
  // groups (with rowsum given, qs is 0 and the total comes off at the end)
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
  auto sum_of = [&](int nl, int tl) {
    const int rt = nl >> 4, i = nl & 15, tt = tl >> 4, j = tl & 15;
    const int slot = (rt * NTT + tt) * 4 + (i & 3);
    const int ln = (i >> 2) * 16 + j;
    int s = 0;
    for (int wv = 0; wv < nwaves; ++wv) s += red[(wv * kSlots + slot) * 64 + ln];
    return derive ? s : s - rowsum[tl];
  };
  if (h) {
    // gated: rows 2i (gate) and 2i + 1 (up) make output n0 / 2 + i
    const float g2 = gamma2[0];
    const int half = N >> 1;
    for (int idx = threadIdx.x; idx < kRows / 2 * kToks; idx += blockDim.x) {
      const int pl = idx % (kRows / 2), tl = idx / (kRows / 2);
      const int n = n0 + 2 * pl;
      if (n >= N || tl >= T) continue;
      const int sg = sum_of(2 * pl, tl), su = sum_of(2 * pl + 1, tl);
      const int64_t o = (int64_t)tl * N + n;
      if (acc_out) {
        acc_out[o] = sg;
        acc_out[o + 1] = su;
      }
      const float a = absmax[tl];
      h[(int64_t)tl * half + (n >> 1)] = gated_relu2_bf16(sg, su, gamma_m(g, a), gamma_m(g2, a));
    }
    return;
  }
  for (int idx = threadIdx.x; idx < kRows * kToks; idx += blockDim.x) {
    const int nl = idx % kRows, tl = idx / kRows;
    const int n = n0 + nl;
    if (n >= N || tl >= T) continue;
    const int s = sum_of(nl, tl);
    const int64_t o = (int64_t)tl * N + n;
    if (acc_out) acc_out[o] = s;
    y[o] = (float)s * out_scale(g, absmax[tl]);
  }
}

// Decode kernel for T <= 16 and K % 256 == 0 (T <= 4 with step A1 fused).
//
// Unpacking: per chunk (256 k of a 16-row tile) a lane holds four packed
// words.  Three of the four 2-bit fields are only masked: w & 0x03030303,
// w & 0x0C0C0C0C and w & 0x30303030 hold c, 4c and 16c in each byte (all
// non-negative int8), and only the top field needs a shift.  Slice j of the
// four words is one MFMA operand; each scale accumulates separately and the
// exact sums are divided by 4 and 16 at the end (they are exact multiples).
// The B operand that matches slice j is dword j of each of the four 16-byte
// activation vectors that cover the lane's 64 k.
//
// A decode launch moves a few MB, so its time is mostly latency:
//  - a block's problem is blockIdx.y, known before the first load, and all
//    arguments arrive in one batch;
//  - the activations are issued first and a block barrier follows before
//    any weight load, so all of a block's activation loads reach memory
//    ahead of all its weight loads (int8 input: global -> LDS directly;
//    one raw token: into registers, four values per lane per chunk; more
//    raw tokens: wave 0 stages the rows in LDS);
//  - wave w owns a contiguous run of at most CPW chunks of its 16 rows and
//    issues all of their loads at once: one memory round trip per wave;
//  - the block barriers wait for LDS traffic only, so the weight loads stay
//    in flight while the activations land (and, with step A1 fused, while
//    they are quantised: every block derives the token absmax itself,
//    scales, rounds half to even and clips exactly as the act-quant kernel
//    does, and block 0 of each problem stores the int8 activations and
//    absmax);
//  - each wave removes the code offset (c = t + 1) of its own k run with the
//    sum of q over that run, computed while its loads are in flight; the
//    waves add their partial tiles in LDS and the last one to finish writes
//    the block's outputs.
enum DecMode { kInt8 = 0, kBf16 = 1, kF32 = 2 };

struct DecProblem {
  const uint32_t* packed;
  const float* gamma;
  const void* x;          // int8 activations (kInt8) or raw bf16 / f32
  const float* absmax;    // kInt8: per-token absmax from act-quant
  float* y;
  int32_t* acc;           // optional exact sums
  int8_t* xq_out;         // fused modes: quantised activations out (block 0)
  float* absmax_out;      // fused modes: absmax out (block 0)
  const float* gamma2;     // gated: the up projection's gamma (gamma is the gate's)
  uint16_t* h;            // gated: [T, N / 2] bfloat16 out (then y is not written)
  int N, K;
  int per;                // chunks per wave: ceil((K / 256) / nw) <= CPW
  int ldy;                // row stride of y and acc (N, or more for a row range of a wider problem)
  const int32_t* rowsum;  // kInt8: each token's sum of q, or NULL (each wave sums its own k run)
};
constexpr int kMaxGroup = 8;
struct DecGroup {
  DecProblem p[kMaxGroup];
  int T, nw;              // tokens; waves per block (the block has 64 * nw threads)
};

// LDS header of the decode kernel: 64 zero bytes, the 16-token x 16 RT-row
// int32 tile (token-major), the finishing counter and 16 absmax bit patterns
// (padded to 16 bytes).
constexpr int dec_head(int rt) { return 64 + 256 * rt * 4 + 4 + 16 * 4 + 12; }
static_assert(dec_head(1) % 16 == 0 && dec_head(2) % 16 == 0, "LDS header alignment");

#ifndef BL_GEMV_DEC_EARLY_DIV
#define BL_GEMV_DEC_EARLY_DIV 4       // CPW / this (at least 1) weight chunks per wave go out early
#endif

// Waves per SIMD the decode kernel is compiled for: eight with int8 input on
// one row tile (64 VGPRs), fewer where the raw activations or a second row
// tile's weights take registers.
constexpr int dec_waves_per_eu(int cpw, int mode, int rt) {
  return rt == 1 ? (mode == 0 ? 8 : 6) : (cpw == 8 ? 4 : cpw == 4 ? 5 : 6);
}

typedef __attribute__((address_space(3))) void* dec_lds_t;
typedef __attribute__((address_space(1))) void* dec_glb_t;

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

// TAIL: some problem's K is not a multiple of 256; the index clamps and
// zeros it needs stay out of the other launches (measured: 1.2% on the 2B
// layer)
template <int CPW, int MODE, bool ONE, bool GATED, int RT, bool TAIL>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(dec_waves_per_eu(CPW, MODE, RT)))) void k_gemv_dec(const DecGroup grp) {
  constexpr int kRows = 16 * RT;                    // weight rows of a block (RT tiles of 16)
  extern __shared__ __align__(16) unsigned char smem[];
  const DecProblem pr = grp.p[blockIdx.y];
  const int T = ONE ? 1 : grp.T, nwaves = grp.nw;
  // Every argument in one batch of scalar loads: without this the compiler
  // fetches them in dependent rounds around the early exit below.
  __asm__ volatile("" ::"s"(pr.packed), "s"(pr.gamma), "s"(pr.x), "s"(pr.absmax), "s"(pr.y),
                   "s"(pr.acc), "s"(pr.xq_out), "s"(pr.absmax_out), "s"(pr.N), "s"(pr.K),
                   "s"(pr.per), "s"(pr.ldy), "s"(pr.rowsum), "s"(T), "s"(nwaves));
  if constexpr (GATED) __asm__ volatile("" ::"s"(pr.gamma2), "s"(pr.h));
  const int N = pr.N, K = pr.K, per = pr.per;
  const int n0 = (int)blockIdx.x * kRows;
  if (n0 >= N) return;                              // the grid spans the widest problem

  const int lane = threadIdx.x & 63, nthreads = nwaves * 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qg = lane >> 4, r = lane & 15;
  const int K16 = K >> 4;
  // 16 words (256 k) per chunk; a row whose K is not a multiple of 256 ends
  // in a short chunk of one to three 64-k quads (K % 64 == 0, host): the
  // lanes of the missing quads load the last valid quad again and meet zero
  // activations
  const int nchunks = (K + 255) >> 8;
  const int c0 = wave * per;
  const int cnt = min(per, nchunks - c0);           // <= 0 when K is narrower than the block

  // LDS: [header][T x (Kp + 16) int8 activations, row-major, Kp = K rounded
  //      up to whole chunks and zero past K; the 16-byte pad per token
  //      spreads the tokens of one B-operand read over the banks]
  //      [fused modes: the raw activations, T x K]
  const int tstride = ((K + 255) & ~255) + 16;
  int* zero = reinterpret_cast<int*>(smem);                    // 16 ints of zeros
  int* tile = zero + 16;                                       // [token][row]
  int* counter = tile + 256 * RT;
  int* amax = counter + 1;
  unsigned char* xs8 = smem + dec_head(RT);
  unsigned char* raw = xs8 + T * tstride;

  const uint4* wrow[RT];                            // row r of each 16-row tile
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    int n = n0 + 16 * rt + r;
    n = n < N ? n : N - 1;                          // rows past N are computed, never stored
    wrow[rt] = reinterpret_cast<const uint4*>(pr.packed + (int64_t)n * K16) + (TAIL ? 0 : qg);
  }
  const int qlast = (K >> 6) - 1;                   // the row's last 64-k quad

  // Issue order matters: vector memory operations retire in order, so what
  // is waited on first goes first.  The token absmax (int8 input) ...
  // (gated outputs: token l >> 3 of lane l, eight outputs per token)
  constexpr bool gated = GATED;
  float am = 0.0f;
  int rsv = 0;   // ... and, given, the token's row sum (both used by the epilogue's first pass)
  if constexpr (MODE == kInt8) {
    const int tl0 = min(lane / (gated ? kRows / 2 : kRows), T - 1);
    am = pr.absmax[tl0];
    if (pr.rowsum) rsv = pr.rowsum[tl0];
  }
  // ... then the activations, straight into LDS (lane l's 16 bytes land at
  // the wave's base + 16 l): int8 input, this wave's own k run; raw input
  // (step A1 fused), the whole rows, shared by the block ...
  const int run0 = c0 * 256, runb = cnt > 0 ? cnt * 256 : 0;   // this wave's k run
  const int runv = TAIL ? (cnt > 0 ? min(runb, K - run0) : 0) : runb;   // ... inside the row
  uint4 xraw[ONE && MODE != kInt8 ? CPW : 1];                  // one-token raw units
  if constexpr (MODE == kInt8) {
    const int8_t* x8 = static_cast<const int8_t*>(pr.x);
    for (int t = 0; t < T; ++t) {
      for (int base = 0; base < runv; base += 1024)
        if (base + 16 * lane < runv)
          __builtin_amdgcn_global_load_lds(
              (dec_glb_t)(x8 + (int64_t)t * K + run0 + base + 16 * lane),
              (dec_lds_t)(xs8 + t * tstride + run0 + base), 16, 0, 0);
      // the end of a row's last chunk past K: zeros (fewer than 256 bytes)
      if (TAIL && run0 + runv + 16 * lane < run0 + runb)
        *reinterpret_cast<uint4*>(xs8 + t * tstride + run0 + runv + 16 * lane) =
            make_uint4(0u, 0u, 0u, 0u);
    }
  } else if constexpr (ONE) {
    // one token: each lane loads, into registers, the four raw activations
    // it will quantise in each chunk of this wave's run (elements 4l .. 4l+3
    // of the chunk); slots past cnt repeat the row's last chunk and feed
    // only the absmax, where a repeat changes nothing
    const unsigned char* xr = static_cast<const unsigned char*>(pr.x);
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      // past K (a short last chunk) the lane loads the row's last four
      // values and takes zeros instead: no branch around the loads
      const int k0 = min(c0 + u, nchunks - 1) * 256 + 4 * lane;
      const int kl = TAIL ? min(k0, K - 4) : k0;
      if constexpr (MODE == kBf16) {
        const uint2 v = *reinterpret_cast<const uint2*>(xr + 2 * kl);
        xraw[u] = make_uint4(v.x, v.y, 0u, 0u);
      } else {
        xraw[u] = *reinterpret_cast<const uint4*>(xr + 4 * kl);
      }
      if (TAIL && k0 != kl) xraw[u] = make_uint4(0u, 0u, 0u, 0u);
    }
  } else {
    const unsigned char* xr = static_cast<const unsigned char*>(pr.x);
    const int nvec = T * K / (MODE == kBf16 ? 8 : 4);
    // wave 0 fetches the whole raw rows (the barrier below puts them ahead
    // of every weight load of the block): shared out over the waves, the
    // fetch takes more instructions and the prologue still waits for all of
    // it (measured: the 2B decode layer 871 -> 923 GB/s before the barrier)
    if (wave == 0) {
      for (int base = 0; base < nvec; base += 64)
        if (base + lane < nvec)
          __builtin_amdgcn_global_load_lds((dec_glb_t)(xr + 16 * (base + lane)),
                                           (dec_lds_t)(raw + 16 * base), 16, 0, 0);
    }
  }
  const float g = pr.gamma[0];
  float g2 = 0.0f;
  if constexpr (GATED) g2 = pr.gamma2[0];
  // A block barrier here, before any weight load, puts every activation
  // load of the block ahead of every weight load of the block in the CU's
  // memory queue, whose loads come back roughly in issue order: the
  // activations, needed first, are no longer stuck behind other waves'
  // weights (measured: the 2B decode layer 920 -> 1005 GB/s, 28672 -> 8192 at
  // one int8 token 15.5 -> 14.4 us).  A wave reaches it as soon as its
  // activation loads are issued; after the weight loads it would wait until
  // all of those are issued, which stalls while the CU's queue is full.  The
  // same barrier orders the header clearing before the tile adds.
  for (int i = threadIdx.x; i < 16 + 256 * RT + 1 + 16; i += nthreads) zero[i] = 0;
  lds_sync();
  // ... and last the weight chunks of this wave; slots past cnt repeat the
  // row's last chunk and meet a zero B operand below.
  uint4 buf[RT][CPW];
  auto issue_w = [&](auto loc, auto hic) {
    constexpr int LO = decltype(loc)::value, HI = decltype(hic)::value;
#pragma unroll
    for (int i = LO; i < HI; ++i) {
      // quad qg of chunk c; in a short last chunk the lanes of the missing
      // quads reload the row's last one
      const int c = min(c0 + i, nchunks - 1);
      const int qi = TAIL ? min(c * 4 + qg, qlast) : c * 4;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) buf[rt][i] = wrow[rt][qi];
    }
  };
  // Only a quarter of the chunks (at least one) go out now, the rest after
  // the activation work: a wave issues in order, and while the CU's memory
  // queue is full, loads are accepted only as data returns, which held the
  // activation work back behind the weight stream (measured: the 2B layer
  // 1192 -> 1208 GB/s with one of two chunks early, 70B 28672 -> 8192 at one
  // int8 token 14.4 -> 14.2 us with two of eight; all chunks early as before,
  // or one of eight, measured the old times).
  constexpr int kE = CPW / BL_GEMV_DEC_EARLY_DIV > 1 ? CPW / BL_GEMV_DEC_EARLY_DIV : 1;
  issue_w(std::integral_constant<int, 0>{}, std::integral_constant<int, kE>{});

  int qsum = 0;     // sum of q over this wave's k run, token of lane l: l & 15
  float a_t = 0.0f; // one raw token: its absmax
  if constexpr (MODE == kInt8) {
    wait_vmem<RT * kE>();                               // this wave's activation run landed
    for (int t = 0; t < (pr.rowsum ? 0 : T); ++t) {     // with rowsum: the totals, at the end
      const uint4* xt = reinterpret_cast<const uint4*>(xs8 + t * tstride + run0);
      int part = 0;
      for (int i = lane; i < runb / 16; i += 64) {
        const uint4 v = xt[i];
        part = __builtin_amdgcn_sdot4((int)v.x, 0x01010101, part, false);
        part = __builtin_amdgcn_sdot4((int)v.y, 0x01010101, part, false);
        part = __builtin_amdgcn_sdot4((int)v.z, 0x01010101, part, false);
        part = __builtin_amdgcn_sdot4((int)v.w, 0x01010101, part, false);
      }
      const int sum = wave_sum_i(part);
      if (r == t) qsum = sum;
    }
  } else if constexpr (ONE) {
    // Step A1 in the block, one token, from registers: the absmax over this
    // wave's run (its repeats included), then over the block through LDS ...
    wait_vmem<RT * kE>();                               // this lane's raw activations landed
    uint32_t mx = 0;                                // magnitude bit patterns
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      const uint4 v = xraw[u];
      if constexpr (MODE == kBf16) {
        typedef unsigned short us2 __attribute__((ext_vector_type(2)));
        const uint32_t m = 0x7fff7fffu;
        const us2 h = __builtin_elementwise_max(__builtin_bit_cast(us2, v.x & m),
                                                __builtin_bit_cast(us2, v.y & m));
        mx = max(mx, (uint32_t)max(h.x, h.y) << 16);
      } else {
        mx = max(mx, max(max(v.x & 0x7fffffffu, v.y & 0x7fffffffu),
                         max(v.z & 0x7fffffffu, v.w & 0x7fffffffu)));
      }
    }
    const int wm = wave_max_nonneg((int)mx);        // non-negative patterns order as values
    if (lane == 0) atomicMax(&amax[0], wm);
    lds_sync();
    // ... then scale, round half to even and clip this lane's units into the
    // int8 row (read back only by this wave: no barrier), summing q.  Block 0
    // of the problem also stores the int8 activations and the absmax.
    const float a = __uint_as_float((uint32_t)amax[0]);
    const float s = kQb / fmaxf(a, kEps);
    a_t = a;
    const bool first = blockIdx.x == 0;
    int tsum = 0;
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      if (u >= cnt) break;                          // wave-uniform
      const int k0 = run0 + u * 256 + 4 * lane;
      const uint4 v = xraw[u];
      float f[4];
      if constexpr (MODE == kBf16) {
        f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
        f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
      } else {
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
      }
      int q[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        q[e] = (int)fminf(fmaxf(rintf(f[e] * s), -kQb), kQb);   // one binary32 product
      const uint32_t lo = __builtin_amdgcn_perm((uint32_t)q[1], (uint32_t)q[0], 0x0c0c0400u);
      const uint32_t hi = __builtin_amdgcn_perm((uint32_t)q[3], (uint32_t)q[2], 0x04000c0cu);
      const uint32_t word = lo | hi;
      tsum = __builtin_amdgcn_sdot4((int)word, 0x01010101, tsum, false);
      *reinterpret_cast<uint32_t*>(xs8 + k0) = word;     // zeros past K
      if (first && pr.xq_out && (!TAIL || k0 < K))
        *reinterpret_cast<uint32_t*>(pr.xq_out + k0) = word;
    }
    const int sum = wave_sum_i(tsum);
    if (r == 0) qsum = sum;
    if (first && wave == 0 && pr.absmax_out && lane == 0) pr.absmax_out[0] = a;
  } else {
    // Step A1 in the block.  The absmax of each token (T <= 4) over all of
    // K, from every wave's share of the raw rows ...
    wait_vmem<RT * kE>();                               // wave 0: the raw rows landed
    lds_sync();                                     // ... for every wave
    constexpr int E = MODE == kBf16 ? 8 : 4;        // elements per 16 bytes
    const int per_tok = K / E, nvec = T * per_tok;
    const uint4* raw4 = reinterpret_cast<const uint4*>(raw);
    uint32_t tmax[4] = {0, 0, 0, 0};                // magnitude bit patterns
    for (int i = threadIdx.x; i < nvec; i += nthreads) {
      const uint4 v = raw4[i];
      uint32_t mx;
      if constexpr (MODE == kBf16) {
        // bf16 magnitudes order as unsigned 16-bit integers: packed max
        typedef unsigned short us2 __attribute__((ext_vector_type(2)));
        const uint32_t m = 0x7fff7fffu;
        us2 h = __builtin_elementwise_max(
            __builtin_bit_cast(us2, v.x & m), __builtin_bit_cast(us2, v.y & m));
        h = __builtin_elementwise_max(h, __builtin_bit_cast(us2, v.z & m));
        h = __builtin_elementwise_max(h, __builtin_bit_cast(us2, v.w & m));
        mx = (uint32_t)max(h.x, h.y) << 16;
      } else {
        mx = max(max(v.x & 0x7fffffffu, v.y & 0x7fffffffu), max(v.z & 0x7fffffffu, v.w & 0x7fffffffu));
      }
      if constexpr (ONE) {
        tmax[0] = max(tmax[0], mx);
      } else {
        const int t = (i >= per_tok) + (i >= 2 * per_tok) + (i >= 3 * per_tok);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
          if (t == tt) tmax[tt] = max(tmax[tt], mx);
      }
    }
#pragma unroll
    for (int tt = 0; tt < (ONE ? 1 : 4); ++tt) {
      if (tt < T) {
        const int wm = wave_max_nonneg((int)tmax[tt]);  // non-negative patterns order as values
        if (lane == 0) atomicMax(&amax[tt], wm);
      }
    }
    lds_sync();
    // ... then each wave scales, rounds half to even and clips its own k run
    // into the int8 rows (read back only by this wave: no barrier), four
    // activations per lane at a time, summing q on the way.  Block 0 of the
    // problem also stores the int8 activations and the absmax.
    float sc[4];
#pragma unroll
    for (int tt = 0; tt < (ONE ? 1 : 4); ++tt)
      sc[tt] = tt < T ? kQb / fmaxf(__uint_as_float((uint32_t)amax[tt]), kEps) : 0.0f;
    const bool first = blockIdx.x == 0;
    const int ru = runb / 4;                        // 4-element units per token in the run
    int tsum[4] = {0, 0, 0, 0};
    for (int i = lane; i < T * ru; i += 64) {
      const int t = ONE ? 0 : (i >= ru) + (i >= 2 * ru) + (i >= 3 * ru);
      const int k0 = run0 + (i - t * ru) * 4;       // first k of the unit
      // a short last chunk: units past K read the row's last four values
      // and quantise zeros instead
      const int kl = TAIL ? min(k0, K - 4) : k0;
      float f[4];
      if constexpr (MODE == kBf16) {
        const uint2 v = *reinterpret_cast<const uint2*>(raw + 2 * ((int64_t)t * K + kl));
        f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
        f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
      } else {
        const uint4 v = *reinterpret_cast<const uint4*>(raw + 4 * ((int64_t)t * K + kl));
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
      }
      if (TAIL && k0 != kl) f[0] = f[1] = f[2] = f[3] = 0.0f;
      float s = sc[0];
      if constexpr (!ONE) {
#pragma unroll
        for (int tt = 1; tt < 4; ++tt)
          if (t == tt) s = sc[tt];
      }
      int q[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        q[e] = (int)fminf(fmaxf(rintf(f[e] * s), -kQb), kQb);   // one binary32 product
      // low bytes of q0..q3 into one word
      const uint32_t lo = __builtin_amdgcn_perm((uint32_t)q[1], (uint32_t)q[0], 0x0c0c0400u);
      const uint32_t hi = __builtin_amdgcn_perm((uint32_t)q[3], (uint32_t)q[2], 0x04000c0cu);
      const uint32_t word = lo | hi;
      const int part = __builtin_amdgcn_sdot4((int)word, 0x01010101, 0, false);
      if constexpr (ONE) {
        tsum[0] += part;
      } else {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
          if (t == tt) tsum[tt] += part;
      }
      *reinterpret_cast<uint32_t*>(xs8 + t * tstride + k0) = word;
      if (first && pr.xq_out && (!TAIL || k0 < K))
        *reinterpret_cast<uint32_t*>(pr.xq_out + (int64_t)t * K + k0) = word;
    }
#pragma unroll
    for (int tt = 0; tt < (ONE ? 1 : 4); ++tt) {
      if (tt < T) {
        const int sum = wave_sum_i(tsum[tt]);
        if (r == tt) qsum = sum;
      }
    }
    if (first && wave == 0 && pr.absmax_out && lane < T)
      pr.absmax_out[lane] = __uint_as_float((uint32_t)amax[lane]);
  }

  // the rest of the weight chunks, after the activation work (a wave issues
  // in order, and loads wait in issue while the CU's memory queue is full)
  issue_w(std::integral_constant<int, kE>{}, std::integral_constant<int, CPW>{});

  // B operands of slot i: this token's 64 bytes of chunk c0 + i (four
  // 16-byte vectors; slice j takes dword j of each), or zeros for tokens past
  // T and for the repeated slots past cnt
  const unsigned char* xrow = xs8 + (r < T ? r : 0) * tstride + qg * 64;
  v4i a1[RT], a4[RT], a16[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) a1[rt] = a4[rt] = a16[rt] = v4i{0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const uint32_t* xc = (r < T && i < cnt)
                             ? reinterpret_cast<const uint32_t*>(xrow + (c0 + i) * 256)
                             : reinterpret_cast<const uint32_t*>(zero);
    // slice j: dword j of each 16-byte vector (two ds_read2_b32 each)
    auto xs = [&](int j) { return v4i{(int)xc[j], (int)xc[4 + j], (int)xc[8 + j], (int)xc[12 + j]}; };
    if constexpr (RT == 1) {
      const uint4 w4 = buf[0][i];
      if constexpr (CPW < 8) {
        // fields masked in place: c, 4c and 16c per byte, three accumulators
        a1[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
            (v4i{(int)(w4.x & 0x03030303u), (int)(w4.y & 0x03030303u), (int)(w4.z & 0x03030303u),
                 (int)(w4.w & 0x03030303u)}),
            xs(0), a1[0], 0, 0, 0);
        a4[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
            (v4i{(int)(w4.x & 0x0C0C0C0Cu), (int)(w4.y & 0x0C0C0C0Cu), (int)(w4.z & 0x0C0C0C0Cu),
                 (int)(w4.w & 0x0C0C0C0Cu)}),
            xs(1), a4[0], 0, 0, 0);
        a16[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
            (v4i{(int)(w4.x & 0x30303030u), (int)(w4.y & 0x30303030u), (int)(w4.z & 0x30303030u),
                 (int)(w4.w & 0x30303030u)}),
            xs(2), a16[0], 0, 0, 0);
      } else {
        // eight chunks in flight leave no room for three accumulators: every
        // field is shifted down to c and summed in one
#pragma unroll
        for (int j = 0; j < 3; ++j)
          a1[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
              (v4i{(int)codes_of(w4.x, j), (int)codes_of(w4.y, j), (int)codes_of(w4.z, j),
                   (int)codes_of(w4.w, j)}),
              xs(j), a1[0], 0, 0, 0);
      }
      a1[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
          (v4i{(int)((w4.x >> 6) & 0x03030303u), (int)((w4.y >> 6) & 0x03030303u),
               (int)((w4.z >> 6) & 0x03030303u), (int)((w4.w >> 6) & 0x03030303u)}),
          xs(3), a1[0], 0, 0, 0);
    } else {
      // two row tiles: the same, slice by slice, one B slice serving both
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v4i b = xs(j);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const uint4 w4 = buf[rt][i];
          v4i a;
          if (j == 3) {
            a = v4i{(int)((w4.x >> 6) & 0x03030303u), (int)((w4.y >> 6) & 0x03030303u),
                    (int)((w4.z >> 6) & 0x03030303u), (int)((w4.w >> 6) & 0x03030303u)};
          } else if constexpr (CPW < 8) {
            const uint32_t m = j == 0 ? 0x03030303u : j == 1 ? 0x0C0C0C0Cu : 0x30303030u;
            a = v4i{(int)(w4.x & m), (int)(w4.y & m), (int)(w4.z & m), (int)(w4.w & m)};
          } else {
            a = v4i{(int)codes_of(w4.x, j), (int)codes_of(w4.y, j), (int)codes_of(w4.z, j),
                    (int)codes_of(w4.w, j)};
          }
          if (CPW < 8 && j == 1)
            a4[rt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, a4[rt], 0, 0, 0);
          else if (CPW < 8 && j == 2)
            a16[rt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, a16[rt], 0, 0, 0);
          else
            a1[rt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, a1[rt], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // one chunk's operands live at a time
  }

  // lane (qg, r) holds rows 16 rt + 4qg + v of token column r
  if (r < T) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        atomicAdd(&tile[r * kRows + 16 * rt + 4 * qg + v],
                  a1[rt][v] + (a4[rt][v] >> 2) + (a16[rt][v] >> 4) - qsum);
  }
  // The last wave to add its tile writes the block's outputs; the others are
  // done.  The counter's release/acquire orders the tile adds before it.
  int ticket = 0;
  if (lane == 0)
    ticket = __hip_atomic_fetch_add(counter, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
  ticket = __builtin_amdgcn_readfirstlane(ticket);
  if (ticket != nwaves - 1) return;
  if constexpr (GATED) {
    // rows 2i (gate) and 2i + 1 (up) of the tile make output n0 / 2 + i
    const int ldy = pr.ldy, half = ldy >> 1;
    for (int idx = lane; idx < kRows / 2 * T; idx += 64) {
      const int i = idx % (kRows / 2), tl = idx / (kRows / 2);
      const int nn = n0 + 2 * i;
      if (nn >= N) continue;
      const int qt = MODE == kInt8 && pr.rowsum ? (idx < 64 ? rsv : pr.rowsum[tl]) : 0;
      const int sg = __hip_atomic_load(&tile[tl * kRows + 2 * i], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP) - qt;
      const int su = __hip_atomic_load(&tile[tl * kRows + 2 * i + 1], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP) - qt;
      if (pr.acc) {
        pr.acc[(int64_t)tl * ldy + nn] = sg;
        pr.acc[(int64_t)tl * ldy + nn + 1] = su;
      }
      float a;
      if constexpr (MODE == kInt8) a = idx < 64 ? am : pr.absmax[tl];
      else a = __uint_as_float((uint32_t)amax[tl]);
      pr.h[(int64_t)tl * half + (nn >> 1)] =
          gated_relu2_bf16(sg, su, gamma_m(g, a), gamma_m(g2, a));
    }
    return;
  }
  for (int idx = lane; idx < kRows * T; idx += 64) {
    const int i = idx % kRows, tl = idx / kRows;
    const int nn = n0 + i;
    if (nn >= N) continue;
    const int sum = __hip_atomic_load(&tile[idx], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) -
                    (MODE == kInt8 && pr.rowsum ? (idx < 64 ? rsv : pr.rowsum[tl]) : 0);
    const int64_t o = (int64_t)tl * pr.ldy + nn;
    if (pr.acc) pr.acc[o] = sum;
    float a;                                        // the token's absmax (int8: lane's own first)
    if constexpr (MODE == kInt8) a = idx < 64 ? am : pr.absmax[tl];
    else a = ONE ? a_t : __uint_as_float((uint32_t)amax[tl]);
    pr.y[o] = (float)sum * out_scale(g, a);
  }
}

#ifndef BL_GEMV_PERSIST_INT8_MAX_K
// One int8 token over many tiles takes the persistent kernel for rows up to
// this long (8192 -> 28672 at one token: 13.1-13.3 -> 12.7 us; on 28672-long
// rows, seven chunks per wave, it measured 14.85 against 14.4 us)
#define BL_GEMV_PERSIST_INT8_MAX_K 8192
#endif
#ifndef BL_GEMV_PERSIST_INT8_MAX_T
#define BL_GEMV_PERSIST_INT8_MAX_T 4    // int8 tokens the persistent kernel takes (at most 4)
#endif
#ifndef BL_GEMV_PERSIST_EARLY
#define BL_GEMV_PERSIST_EARLY 2         // weight chunks per wave issued ahead of step A1
#endif

// Persistent decode kernel for one token over many 16-row tiles (the
// 70B-class shapes, hundreds to thousands of tiles), raw (bf16 / f32, step
// A1 fused) or int8: a grid of a few blocks per CU, each block taking tiles b, b + G,
// b + 2G, ... (G blocks), so that the tiles read at any moment are
// neighbours in memory.  The block's waves split K as in k_gemv_dec (wave w
// owns chunks w*per .. w*per+per-1 of every tile), but the token is fetched
// and quantised once per block instead of once per tile, each wave's sum of
// q over its k run is formed once, and every wave keeps the weight loads of
// its next DEPTH - 1 tiles in flight while it contracts the current one,
// chunk by chunk as they land.  Each tile has its own LDS slot (16 partial
// sums and a counter); the last wave to add into it writes the tile's 16
// outputs.  On int8 input the codes are copied into the row as they are
// (with the token's row sum, if given, subtracted once); there it serves
// rows of up to 8192 only (longer rows measured faster with k_gemv_dec's
// block per tile).
//
// The int8 row sits in LDS slice-major: chunk c, lane group qg, slice j
// hold the four dwords {4u + j : u = 0..3} of the group's 64 k, so one
// ds_read_b128 is one MFMA B operand.  Each wave writes and reads only its
// own k run (no block barrier between them).
constexpr int persist_head(int tpb, int nt) {
  return ((16 + (16 * nt + 1) * tpb + 1) * 4 + 15) / 16 * 16;
}

// byte offset, in a chunk's 256 bytes, of dword d (k = 4d .. 4d + 3) in the
// slice-major order
__device__ __forceinline__ int slice_off(int d) {
  return (d >> 4) * 64 + (d & 3) * 16 + ((d >> 2) & 3) * 4;
}

// Calls f(integral_constant<int, J>) for J = 0 .. sizeof...(J) - 1, in order.
template <class F, int... J>
__device__ __forceinline__ void for_each_c(F&& f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>{}), ...);
}

// HOLD_B: the B operands (the wave's int8 activations, the same for every
// tile) may stay in registers across tiles; otherwise they are read from LDS
// again for every tile (long K: 16 registers per chunk would not fit).
// NT: int8 input only, one to four tokens; token t's row is its own
// slice-major row in LDS, lanes (qg, r) of token column r < NT read it, and a
// tile's partial sums hold 16 rows per token.
template <int CPW, int MODE, int DEPTH, bool HOLD_B, int NT>
__global__ __launch_bounds__(1024) void k_gemv_persist(const DecProblem pr, int nwaves, int tpb) {
  static_assert(DEPTH >= 2 && DEPTH <= 4 && DEPTH * CPW < 64, "tiles in flight");
  static_assert(NT == 1 || (MODE == kInt8 && NT <= 4), "several tokens: int8 input, at most four");
  extern __shared__ __align__(16) unsigned char smem[];
  __asm__ volatile("" ::"s"(pr.packed), "s"(pr.gamma), "s"(pr.x), "s"(pr.absmax), "s"(pr.y),
                   "s"(pr.acc), "s"(pr.xq_out), "s"(pr.absmax_out), "s"(pr.N), "s"(pr.K),
                   "s"(pr.per), "s"(pr.rowsum), "s"(nwaves), "s"(tpb));
  const int N = pr.N, K = pr.K, per = pr.per;
  const int G = gridDim.x, b = blockIdx.x;
  const int tiles = (N + 15) >> 4;
  const int ntb = (tiles - b + G - 1) / G;          // this block's tiles: DEPTH <= ntb <= tpb (host)
  const int lane = threadIdx.x & 63, nthreads = nwaves * 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qg = lane >> 4, r = lane & 15;
  const int K16 = K >> 4;
  const int nchunks = K >> 8;
  const int c0 = wave * per;
  const int cnt = min(per, nchunks - c0);           // >= 1: the host sizes nwaves to the chunks

  // LDS: 16 zero ints | tpb x 16 NT partial sums | tpb counters | absmax bits |
  //      NT int8 rows of K
  int* zero = reinterpret_cast<int*>(smem);
  int* slot = zero + 16;
  int* counter = slot + 16 * NT * tpb;
  int* amax = counter + tpb;
  unsigned char* xs8 = smem + persist_head(tpb, NT);

  // the raw token first (vector memory returns in issue order): the four
  // values per chunk this lane quantises, into registers (slots past cnt
  // repeat the row's last chunk and feed only the absmax)
  const int run0 = c0 * 256;
  uint4 xin[CPW];
  {
    const unsigned char* xr = static_cast<const unsigned char*>(pr.x);
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      const int k0 = min(c0 + u, nchunks - 1) * 256 + 4 * lane;
      if constexpr (MODE == kInt8) {
        // token t's four codes in component t
        uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int t = 0; t < NT; ++t) c[t] = *reinterpret_cast<const uint32_t*>(xr + (int64_t)t * K + k0);
        xin[u] = make_uint4(c[0], c[1], c[2], c[3]);
      } else if constexpr (MODE == kBf16) {
        const uint2 v = *reinterpret_cast<const uint2*>(xr + 2 * k0);
        xin[u] = make_uint4(v.x, v.y, 0u, 0u);
      } else {
        xin[u] = *reinterpret_cast<const uint4*>(xr + 4 * k0);
      }
    }
  }
  const float g = pr.gamma[0];
  // int8 input: the absmax of the token whose outputs this lane writes
  // (token lane / 16), and, given, the row sum of its token column r
  float a_in = 0.0f;
  int rs_in = 0;
  if constexpr (MODE == kInt8) {
    a_in = pr.absmax[min(lane >> 4, NT - 1)];
    if (pr.rowsum) rs_in = pr.rowsum[min(r, NT - 1)];
  }
  for (int i = threadIdx.x; i < 16 + (16 * NT + 1) * tpb + 1; i += nthreads) zero[i] = 0;
  lds_sync();   // every activation load of the block is issued ahead of every weight load

  // weight loads of one tile into buffer D: this lane's 16 bytes of each of
  // the wave's chunks (slots past cnt repeat the row's last chunk and meet a
  // zero B operand)
  uint4 buf[DEPTH][CPW];
  // chunks LO .. HI - 1 of tile it into buffer D
  auto issue_part = [&](auto dc, int it, auto loc, auto hic) {
    constexpr int D = decltype(dc)::value, LO = decltype(loc)::value, HI = decltype(hic)::value;
    int n = 16 * (b + it * G) + r;
    n = n < N ? n : N - 1;                          // rows past N are computed, never stored
    const uint4* wr = reinterpret_cast<const uint4*>(pr.packed + (int64_t)n * K16) + qg;
#pragma unroll
    for (int i = LO; i < HI; ++i) buf[D][i] = wr[(size_t)min(c0 + i, nchunks - 1) * 4];
  };
  using C0 = std::integral_constant<int, 0>;
  using CW = std::integral_constant<int, CPW>;
  auto issue = [&](auto dc, int it) { issue_part(dc, it, C0{}, CW{}); };
  // A few chunks of the first tile go ahead of step A1, the rest after it.
  // A wave issues its instructions in order, and while the CU's memory queue
  // is full (every wave asking for DEPTH x CPW weight vectors at once) loads
  // are accepted only as data returns: with all of them issued first, every
  // wave's absmax and quantisation waited behind the weight stream (one bf16
  // row of 28672: the block's absmax done at a median of 9.3 us into the
  // kernel, against 1.6 us now).  The early chunks keep HBM busy meanwhile.
  constexpr int kEarly = BL_GEMV_PERSIST_EARLY < CPW ? BL_GEMV_PERSIST_EARLY : CPW;
  using CE = std::integral_constant<int, kEarly>;
  issue_part(std::integral_constant<int, 0>{}, 0, C0{}, CE{});

  // step A1 once per block: the token absmax over every wave's raw values
  // (repeats included, which change nothing), then each lane quantises its
  // own values into the wave's run of the int8 row in LDS (slice-major),
  // summing q (lanes of token column 0)
  int qsum = 0;
  float a_t;
  wait_vmem<kEarly>();                              // the raw loads landed
  if constexpr (MODE == kInt8) {
    // int8 input: the codes go into the wave's run of the row as they are;
    // the sum of q over the run unless the token's row sum is given
    a_t = a_in;
    int tsum[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) tsum[t] = 0;
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      if (u >= cnt) break;                          // wave-uniform
      const uint32_t words[4] = {xin[u].x, xin[u].y, xin[u].z, xin[u].w};
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        tsum[t] = __builtin_amdgcn_sdot4((int)words[t], 0x01010101, tsum[t], false);
        *reinterpret_cast<uint32_t*>(xs8 + t * K + run0 + u * 256 + slice_off(lane)) = words[t];
      }
    }
    if (pr.rowsum) {
      if (wave == 0 && r < NT) qsum = rs_in;       // each total once, on one wave's lanes
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int sum = wave_sum_i(tsum[t]);
        if (r == t) qsum = sum;
      }
    }
  } else {
    uint32_t mx = 0;
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      const uint4 v = xin[u];
      if constexpr (MODE == kBf16) {
        typedef unsigned short us2 __attribute__((ext_vector_type(2)));
        const uint32_t m = 0x7fff7fffu;
        const us2 h = __builtin_elementwise_max(__builtin_bit_cast(us2, v.x & m),
                                                __builtin_bit_cast(us2, v.y & m));
        mx = max(mx, (uint32_t)max(h.x, h.y) << 16);
      } else {
        mx = max(mx, max(max(v.x & 0x7fffffffu, v.y & 0x7fffffffu),
                         max(v.z & 0x7fffffffu, v.w & 0x7fffffffu)));
      }
    }
    const int wm = wave_max_nonneg((int)mx);
    if (lane == 0) atomicMax(&amax[0], wm);
    lds_sync();
    a_t = __uint_as_float((uint32_t)amax[0]);
    const float s = kQb / fmaxf(a_t, kEps);
    const bool first = b == 0;
    int tsum = 0;
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      if (u >= cnt) break;                          // wave-uniform
      const int k0 = run0 + u * 256 + 4 * lane;
      const uint4 v = xin[u];
      float f[4];
      if constexpr (MODE == kBf16) {
        f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
        f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
      } else {
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
      }
      int q[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        q[e] = (int)fminf(fmaxf(rintf(f[e] * s), -kQb), kQb);   // one binary32 product
      const uint32_t lo = __builtin_amdgcn_perm((uint32_t)q[1], (uint32_t)q[0], 0x0c0c0400u);
      const uint32_t hi = __builtin_amdgcn_perm((uint32_t)q[3], (uint32_t)q[2], 0x04000c0cu);
      const uint32_t word = lo | hi;
      tsum = __builtin_amdgcn_sdot4((int)word, 0x01010101, tsum, false);
      *reinterpret_cast<uint32_t*>(xs8 + run0 + u * 256 + slice_off(lane)) = word;
      if (first && pr.xq_out) *reinterpret_cast<uint32_t*>(pr.xq_out + k0) = word;
    }
    const int sum = wave_sum_i(tsum);
    if (r == 0) qsum = sum;
    if (first && wave == 0 && pr.absmax_out && lane == 0) pr.absmax_out[0] = a_t;
  }
  const float sc = out_scale(g, a_t);
  // the rest of the first DEPTH tiles' weight loads (chunk order per wave
  // unchanged, which the waits below count on)
  issue_part(std::integral_constant<int, 0>{}, 0, CE{}, CW{});
  for_each_c([&](auto dc) {
    if constexpr (decltype(dc)::value > 0) issue(dc, decltype(dc)::value);
  }, std::make_integer_sequence<int, DEPTH>{});

  // one tile: contract each chunk as its loads land, add the partial sums
  // (the last wave to add writes the outputs), then, with REFILL, issue the
  // loads of tile it + DEPTH into the freed buffer.  WAIT is the number of
  // this wave's loads of later tiles in flight.  The refill is never
  // conditional inside a step: the compiler's own waits after a branch that
  // may or may not have issued loads assume the worst and would wait for the
  // loads just issued.
  // (always inlined: an outlined step, seen at seven chunks per wave, keeps
  // its weight buffers in scratch memory)
  auto step = [&](auto dc, auto wc, auto rc, int it) __attribute__((always_inline)) {
    constexpr int D = decltype(dc)::value;
    constexpr int WAIT = decltype(wc)::value;
    constexpr bool REFILL = decltype(rc)::value;
    if constexpr (!HOLD_B) __asm__ volatile("" ::: "memory");   // read B from LDS again
    v4i a1 = {0, 0, 0, 0}, a4 = {0, 0, 0, 0}, a16 = {0, 0, 0, 0};
    for_each_c([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      wait_vmem<WAIT + CPW - 1 - i>();              // chunk i of this tile landed
      const unsigned char* xb = (r < NT && i < cnt) ? xs8 + (r * K + run0 + i * 256 + qg * 64)
                                                    : reinterpret_cast<const unsigned char*>(zero);
      auto xs = [&](int j) {
        return *reinterpret_cast<const v4i*>(xb + ((r < NT && i < cnt) ? 16 * j : 0));
      };
      const uint4 w4 = buf[D][i];
      a1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(
          (v4i{(int)(w4.x & 0x03030303u), (int)(w4.y & 0x03030303u), (int)(w4.z & 0x03030303u),
               (int)(w4.w & 0x03030303u)}),
          xs(0), a1, 0, 0, 0);
      a4 = __builtin_amdgcn_mfma_i32_16x16x64_i8(
          (v4i{(int)(w4.x & 0x0C0C0C0Cu), (int)(w4.y & 0x0C0C0C0Cu), (int)(w4.z & 0x0C0C0C0Cu),
               (int)(w4.w & 0x0C0C0C0Cu)}),
          xs(1), a4, 0, 0, 0);
      a16 = __builtin_amdgcn_mfma_i32_16x16x64_i8(
          (v4i{(int)(w4.x & 0x30303030u), (int)(w4.y & 0x30303030u), (int)(w4.z & 0x30303030u),
               (int)(w4.w & 0x30303030u)}),
          xs(2), a16, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(
          (v4i{(int)((w4.x >> 6) & 0x03030303u), (int)((w4.y >> 6) & 0x03030303u),
               (int)((w4.z >> 6) & 0x03030303u), (int)((w4.w >> 6) & 0x03030303u)}),
          xs(3), a1, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }, std::make_integer_sequence<int, CPW>{});
    if constexpr (REFILL) issue(dc, it + DEPTH);   // ahead of the epilogue's LDS and store work
    // lane (qg, r) holds rows 4qg + v of token r
    if (r < NT) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        atomicAdd(&slot[16 * NT * it + 16 * r + 4 * qg + v],
                  a1[v] + (a4[v] >> 2) + (a16[v] >> 4) - qsum);
    }
    int ticket = 0;
    if (lane == 0)
      ticket = __hip_atomic_fetch_add(&counter[it], 1, __ATOMIC_ACQ_REL,
                                      __HIP_MEMORY_SCOPE_WORKGROUP);
    ticket = __builtin_amdgcn_readfirstlane(ticket);
    if (ticket == nwaves - 1 && lane < 16 * NT) {   // token lane / 16, row lane % 16
      const int n = 16 * (b + it * G) + (lane & 15);
      if (n < N) {
        const int sum = __hip_atomic_load(&slot[16 * NT * it + lane], __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_WORKGROUP);
        const int64_t o = (int64_t)(lane >> 4) * N + n;
        if (pr.acc) pr.acc[o] = sum;
        pr.y[o] = (float)sum * sc;
      }
    }
  };
  // steady state: every step refills (tile it + DEPTH exists), and DEPTH - 1
  // later tiles are in flight at each wait ...
  int it = 0;
  for (; it + 2 * DEPTH - 1 < ntb; it += DEPTH)
    for_each_c([&](auto dc) {
      step(dc, std::integral_constant<int, (DEPTH - 1) * CPW>{}, std::true_type{},
           it + decltype(dc)::value);
    }, std::make_integer_sequence<int, DEPTH>{});
  // ... then the last R tiles (DEPTH <= R < 2 DEPTH), straight-line: step j
  // refills while tile j + DEPTH exists and waits for the tiles after it
  auto tail = [&](auto rc) {
    constexpr int R = decltype(rc)::value;
    for_each_c([&](auto jc) {
      constexpr int J = decltype(jc)::value;
      constexpr int AFTER = R - 1 - J < DEPTH - 1 ? R - 1 - J : DEPTH - 1;
      step(std::integral_constant<int, J % DEPTH>{}, std::integral_constant<int, AFTER * CPW>{},
           std::integral_constant<bool, (J + DEPTH < R)>{}, it + J);
    }, std::make_integer_sequence<int, R>{});
  };
  const int left = ntb - it;
  if (left == DEPTH) tail(std::integral_constant<int, DEPTH>{});
  else if (left == DEPTH + 1) tail(std::integral_constant<int, DEPTH + 1>{});
  else if constexpr (DEPTH >= 3) {
    if (left == DEPTH + 2) tail(std::integral_constant<int, DEPTH + 2>{});
    else if constexpr (DEPTH >= 4) { if (left == DEPTH + 3) tail(std::integral_constant<int, DEPTH + 3>{}); }
  }
}

// Launch-shape tunables (compile-time so variants can be built and compared).
#ifndef BL_GEMV_U
#define BL_GEMV_U 2          // chunks whose loads a wave issues together (6912 -> 2560
                             // at T = 8: 6.0 us with 4, 5.7 with 2, 6.3 with 8)
#endif
#ifndef BL_GEMV_MAXW
#define BL_GEMV_MAXW 8       // most waves per block (they split K)
#endif
#ifndef BL_GEMV_RT2_MIN_BLOCKS
#define BL_GEMV_RT2_MIN_BLOCKS 128   // 32-row blocks for 16 < T <= 64 from this many on
#endif

template <int VEC, int RT, int NTT, int U>
void run(const uint8_t* packed, const float* gamma, const int8_t* xq, const float* absmax,
         const int32_t* rowsum, int t, int n, int k, float* y, int32_t* acc, const float* gamma2,
         uint16_t* h, hipStream_t stream) {
  const int k16 = k / 16;
  const int nchunks = (k16 + 4 * VEC - 1) / (4 * VEC);
  int nw = (nchunks + U - 1) / U;       // one pass of U chunks per wave where possible
  if (nw < 1) nw = 1;
  if (nw > BL_GEMV_MAXW) nw = BL_GEMV_MAXW;
  const int grid = (n + 16 * RT - 1) / (16 * RT);
  const size_t lds = (size_t)nw * RT * NTT * 4 * 64 * sizeof(int);
  k_gemv<VEC, RT, NTT, U><<<grid, nw * 64, lds, stream>>>(
      reinterpret_cast<const uint32_t*>(packed), gamma, xq, absmax, t, n, k, y, acc, gamma2, h,
      rowsum);
}

template <int VEC>
void run_tokens(const uint8_t* packed, const float* gamma, const int8_t* xq,
                const float* absmax, const int32_t* rs, int t, int n, int k, float* y,
                int32_t* acc, const float* gamma2, uint16_t* h, hipStream_t stream) {
  if (t <= 16)
    run<VEC, 1, 1, BL_GEMV_U>(packed, gamma, xq, absmax, rs, t, n, k, y, acc, gamma2, h, stream);
  else if (n < 32 * BL_GEMV_RT2_MIN_BLOCKS) {
    // two-tile blocks would leave most CUs idle: one tile per block, twice
    // the blocks (measured at 6912 -> 2560: T = 32 14.0 -> 11.4 us, T = 64
    // 21.5 -> 17.7 us; at 2560 -> 6912, 216 two-tile blocks, one tile loses)
    if (t <= 32)
      run<VEC, 1, 2, (BL_GEMV_U > 2 ? 2 : BL_GEMV_U)>(packed, gamma, xq, absmax, rs, t, n, k, y,
                                                      acc, gamma2, h, stream);
    else
      run<VEC, 1, 4, 1>(packed, gamma, xq, absmax, rs, t, n, k, y, acc, gamma2, h, stream);
  } else if (t <= 32)
    run<VEC, 2, 2, (BL_GEMV_U > 2 ? 2 : BL_GEMV_U)>(packed, gamma, xq, absmax, rs, t, n, k, y, acc,
                                                    gamma2, h, stream);
  else
    run<VEC, 2, 4, 1>(packed, gamma, xq, absmax, rs, t, n, k, y, acc, gamma2, h, stream);
}

}  // namespace

namespace {

#ifndef BL_GEMV_DEC_RESIDENT
#define BL_GEMV_DEC_RESIDENT 16384  // most waves per launch (two rounds of 8 per SIMD on 1024 SIMDs)
#endif
#ifndef BL_GEMV_DEC_MAXW
#define BL_GEMV_DEC_MAXW 8          // waves per block, unless K needs more (8 chunks each) ...
#endif
#ifndef BL_GEMV_DEC_MAXW_SHORT
#define BL_GEMV_DEC_MAXW_SHORT 16   // ... or this many give every wave BL_GEMV_DEC_CPW chunks
#endif
#ifndef BL_GEMV_DEC_RT2_MIN_TILES
#define BL_GEMV_DEC_RT2_MIN_TILES 512   // 16-row tiles from which a block takes two ...
#endif
#ifndef BL_GEMV_DEC_RT2_MIN_TILES_MULTI
#define BL_GEMV_DEC_RT2_MIN_TILES_MULTI 256   // ... or this many when T > 1 ...
#endif
#ifndef BL_GEMV_DEC_RT2_MAX_CHUNKS
#define BL_GEMV_DEC_RT2_MAX_CHUNKS 16   // ... of rows of at most this many 256-k chunks
#endif
#ifndef BL_GEMV_DEC_CPW
#define BL_GEMV_DEC_CPW 2           // chunks per wave aimed for
#endif
#ifndef BL_GEMV_DEC_XLDS
#define BL_GEMV_DEC_XLDS 32768    // largest T*K of int8 activations staged in LDS
#endif
#ifndef BL_GEMV_DEC_XLDS_FEW
// ... and at up to four int8 tokens, whose long rows would otherwise take
// the 64-token kernel (28672 -> 8192 at T = 2 / 4: 22.0 / 23.9 -> 14.8 /
// 17.7 us; from T = 8 on the larger staging measured slower or equal, e.g.
// 8192 -> 28672 at T = 12 33.3 against 47.7 us, one block per CU)
#define BL_GEMV_DEC_XLDS_FEW 131072
#endif
#ifndef BL_GEMV_DEC_RAWLDS
#define BL_GEMV_DEC_RAWLDS 32768  // largest raw activation bytes (fused act-quant) in LDS
#endif
#ifndef BL_GEMV_FUSE_MAX_WORK
#define BL_GEMV_FUSE_MAX_WORK (4 << 20)   // largest sum of blocks x K quantised in fused launches
#endif
#ifndef BL_GEMV_FUSE_MAX_WORK_T1
#define BL_GEMV_FUSE_MAX_WORK_T1 (16 << 20)   // the same for one token
#endif

// Launch shape of the decode kernel for a group of `blocks` 16-row tiles
// whose widest K is kmax: nw waves per block, each owning at most cpw
// (a template size: 2, 4 or 8) consecutive 256-k chunks.  A block's time is
// mostly latency plus the work its waves do one after another on the SIMDs,
// so: about BL_GEMV_DEC_CPW chunks per wave (up to BL_GEMV_DEC_MAXW_SHORT
// waves per block when that is enough, else at most BL_GEMV_DEC_MAXW), no
// more than BL_GEMV_DEC_RESIDENT waves in all, never more than 8 chunks per
// wave (K <= 32768, 128 chunks, keeps nw <= 16) and no wave without chunks.
// Measured on the 2B layer and the 70B shapes after the block barrier moved
// ahead of the weight loads: 14 waves of 2 chunks for K = 6912 (+0.6% on the
// layer against 8 of 4); 8 of 4 for K = 8192 at 1792 blocks (the fused
// launch 16.8 -> 15.8 us against 4 of 8); 14 of 8 for K = 28672 (16 of 7:
// 15.1 against 14.5 us).
struct DecShape {
  int nw, cpw, rt;          // waves per block, chunks per wave (template), 16-row tiles per block
};
DecShape dec_shape(int64_t tiles, int64_t kmax, int64_t t) {
  // Two row tiles per block for short rows once that still leaves a block
  // for every CU: the block's activations (fetched and, fused, quantised once
  // per block) then serve 32 rows, and half as many blocks are launched.
  // Measured: the 2B gate/up launch (K = 2560, 864 tiles) gains, the layer
  // 1167 -> 1184 GB/s; 70B rows (K = 8192, 28672) lose 2 us, their waves
  // then holding twice the weights at half the occupancy.
  // Several tokens stage T times the activations per block, so two tiles
  // pay from fewer tiles on (measured: 2560 -> 6912 at T = 8, 432 tiles,
  // 6.1 -> 5.7 us; at T = 1 the same change costs 1.5%).
  const int nchunks = (int)((kmax + 255) / 256);
  const int64_t min_tiles = t > 1 ? BL_GEMV_DEC_RT2_MIN_TILES_MULTI : BL_GEMV_DEC_RT2_MIN_TILES;
  const int rt = tiles >= min_tiles && nchunks <= BL_GEMV_DEC_RT2_MAX_CHUNKS ? 2 : 1;
  const int64_t blocks = (tiles + rt - 1) / rt;
  int nw = (nchunks + BL_GEMV_DEC_CPW - 1) / BL_GEMV_DEC_CPW;
  const int maxw = nw <= BL_GEMV_DEC_MAXW_SHORT ? BL_GEMV_DEC_MAXW_SHORT : BL_GEMV_DEC_MAXW;
  if (nw > maxw) nw = maxw;
  const int64_t fit = BL_GEMV_DEC_RESIDENT / blocks;
  if (nw > fit) nw = (int)(fit > 1 ? fit : 1);
  const int least = (nchunks + 7) / 8;
  if (nw < least) nw = least;
  const int per = (nchunks + nw - 1) / nw;
  nw = (nchunks + per - 1) / per;   // the same chunks per wave, no wave left without
  return DecShape{nw, per <= 2 ? 2 : per <= 4 ? 4 : 8, rt};
}

// Shapes the decode kernel takes: raw_bytes is 0 for int8 activations, else
// the size of one raw activation (step A1 fused, at most 4 tokens; one token
// keeps its raw activations in registers, more are staged in LDS).
bool dec_shape_ok(int64_t t, int64_t k, int raw_bytes) {
  // rows of whole 64-k quads (those not a multiple of 256 end in a short
  // chunk)
  const int64_t kp = (k + 255) / 256 * 256;
  // at most 128 chunks: 16 waves of at most 8
  if ((k % 64) != 0 || kp > 32768) return false;
  if (raw_bytes == 0)
    return t <= 16 && (t * kp <= BL_GEMV_DEC_XLDS || (t <= 4 && t * kp <= BL_GEMV_DEC_XLDS_FEW));
  if (t * kp > BL_GEMV_DEC_XLDS) return false;
  return t == 1 || (t <= 4 && t * k * raw_bytes <= BL_GEMV_DEC_RAWLDS);
}

// Fused launches redo the token absmax in every block: worth it while that
// redundant work costs less than a separate act-quant launch.  Measured on
// 8192-wide rows: at one token fusing wins up to 1792 blocks (14.7M staged
// elements; 16.4 against 18.5 us), at two tokens it loses there.
bool fuse_work_ok(int64_t t, int64_t work) {
  return work <= (t == 1 ? BL_GEMV_FUSE_MAX_WORK_T1 : BL_GEMV_FUSE_MAX_WORK);
}

size_t dec_lds(int64_t t, int64_t kmax, int raw_bytes, int rt) {
  const size_t staged = t == 1 ? 0 : (size_t)t * kmax * raw_bytes;   // raw rows, T > 1
  return dec_head(rt) + (size_t)t * ((kmax + 255) / 256 * 256 + 16) + staged;
}

template <int MODE, bool ONE, bool GATED, int RT, bool TAIL>
void launch_dec_cpw(const DecGroup& grp, dim3 grid, const DecShape& sh, size_t lds,
                    hipStream_t stream) {
  if (sh.cpw == 2)
    k_gemv_dec<2, MODE, ONE, GATED, RT, TAIL><<<grid, sh.nw * 64, lds, stream>>>(grp);
  else if (sh.cpw == 4)
    k_gemv_dec<4, MODE, ONE, GATED, RT, TAIL><<<grid, sh.nw * 64, lds, stream>>>(grp);
  else
    k_gemv_dec<8, MODE, ONE, GATED, RT, TAIL><<<grid, sh.nw * 64, lds, stream>>>(grp);
}

template <int MODE, bool ONE, bool GATED, int RT>
void launch_dec_rt(const DecGroup& grp, int count, dim3 grid, const DecShape& sh, size_t lds,
                   hipStream_t stream) {
  bool tail = false;
  for (int i = 0; i < count; ++i) tail = tail || (grp.p[i].K % 256) != 0;
  if (tail) return launch_dec_cpw<MODE, ONE, GATED, RT, true>(grp, grid, sh, lds, stream);
  launch_dec_cpw<MODE, ONE, GATED, RT, false>(grp, grid, sh, lds, stream);
}

template <int MODE, bool ONE, bool GATED>
void launch_dec(const DecGroup& grp, int count, dim3 grid, const DecShape& sh, size_t lds,
                hipStream_t stream) {
  if (sh.rt == 2)
    launch_dec_rt<MODE, ONE, GATED, 2>(grp, count, grid, sh, lds, stream);
  else
    launch_dec_rt<MODE, ONE, GATED, 1>(grp, count, grid, sh, lds, stream);
}

template <int MODE>
hipError_t run_dec(DecGroup& grp, int count, const DecShape& sh, size_t lds,
                   hipStream_t stream) {
  grp.nw = sh.nw;
  int bx = 0;   // blocks of the problem with the most rows
  for (int i = 0; i < count; ++i) {
    grp.p[i].per = ((grp.p[i].K + 255) / 256 + sh.nw - 1) / sh.nw;
    if (grp.p[i].ldy == 0) grp.p[i].ldy = grp.p[i].N;
    const int b = (grp.p[i].N + 16 * sh.rt - 1) / (16 * sh.rt);
    bx = b > bx ? b : bx;
  }
  const dim3 grid((unsigned)bx, (unsigned)count);
  bool one = false;   // single-token specialisation of the fused prologue
  if constexpr (MODE != kInt8) one = grp.T == 1;
  // gated epilogue: a group of one problem with h set (launch_gated)
  if (grp.p[0].h != nullptr) {
    if (one)
      launch_dec<MODE, MODE != kInt8, true>(grp, count, grid, sh, lds, stream);
    else
      launch_dec<MODE, false, true>(grp, count, grid, sh, lds, stream);
  } else if (one) {
    launch_dec<MODE, MODE != kInt8, false>(grp, count, grid, sh, lds, stream);
  } else {
    launch_dec<MODE, false, false>(grp, count, grid, sh, lds, stream);
  }
  return hipGetLastError();
}

#ifndef BL_GEMV_PERSIST_MIN_TILES
#define BL_GEMV_PERSIST_MIN_TILES 512   // 16-row tiles from which one token takes the persistent kernel
#endif
#ifndef BL_GEMV_PERSIST_BPC
#define BL_GEMV_PERSIST_BPC 2           // blocks per CU
#endif
#ifndef BL_GEMV_PERSIST_CPW
#define BL_GEMV_PERSIST_CPW 2           // 256-k chunks per wave aimed for (at most 16 waves)
#endif
constexpr int kPersistMaxK = 28672;     // at most 7 chunks per wave at 16 waves
// Tiles per block at most: the LDS header holds 17 ints per tile of the block
// (with the staged row, 4.4 KB + K per block at 64 tiles).
constexpr int kPersistMaxTpb = 64;

bool persist_ok(int64_t t, int64_t n, int64_t k) {
  const int64_t tiles = (n + 15) / 16;
  return t == 1 && k % 256 == 0 && k <= kPersistMaxK && tiles >= BL_GEMV_PERSIST_MIN_TILES &&
         tiles <= (int64_t)device_cus() * BL_GEMV_PERSIST_BPC * kPersistMaxTpb;
}

// Tiles in flight per wave and whether the B operands stay in registers, by
// chunks per wave: about 128 KiB of weight loads in flight per CU at 16 waves.
#ifndef BL_GEMV_PERSIST_DEPTH
#define BL_GEMV_PERSIST_DEPTH 2         // tiles in flight per wave; 0: by chunks per wave
#endif
constexpr int persist_depth(int cpw) {
  return BL_GEMV_PERSIST_DEPTH ? (BL_GEMV_PERSIST_DEPTH * cpw < 64 ? BL_GEMV_PERSIST_DEPTH : 2)
                               : cpw <= 2 ? 4 : cpw <= 4 ? 3 : 2;
}

template <int MODE, int CPW, int NT = 1>
hipError_t launch_persist_cpw(const DecProblem& pr, int g, int nw, int tpb, size_t lds,
                              hipStream_t stream) {
  k_gemv_persist<CPW, MODE, persist_depth(CPW), (CPW <= 2), NT>
      <<<g, nw * 64, lds, stream>>>(pr, nw, tpb);
  return hipGetLastError();
}

// One raw token, or one to four int8 tokens with at most 32 chunks per row
// (nt), one problem (plain outputs), many tiles: the persistent kernel.
template <int MODE>
hipError_t run_persist(DecProblem pr, hipStream_t stream, int nt = 1) {
  const int tiles = (pr.N + 15) / 16, nchunks = pr.K / 256;
  int per = BL_GEMV_PERSIST_CPW;
  if ((nchunks + per - 1) / per > 16) per = (nchunks + 15) / 16;
  const int nw = (nchunks + per - 1) / per;
  pr.per = per;
  const int cpw = per <= 2 ? 2 : per <= 4 ? 4 : 7;
  int g = device_cus() * BL_GEMV_PERSIST_BPC;
  if (g > tiles / persist_depth(cpw)) g = tiles / persist_depth(cpw);   // DEPTH tiles per block at least
  const int tpb = (tiles + g - 1) / g;
  const size_t lds = persist_head(tpb, nt) + (size_t)nt * pr.K;
  if constexpr (MODE == kInt8) {
    if (nt > 1 && cpw != 2) return hipErrorInvalidValue;   // the host keeps K <= 8192
    if (nt == 2) return launch_persist_cpw<MODE, 2, 2>(pr, g, nw, tpb, lds, stream);
    if (nt == 3) return launch_persist_cpw<MODE, 2, 3>(pr, g, nw, tpb, lds, stream);
    if (nt == 4) return launch_persist_cpw<MODE, 2, 4>(pr, g, nw, tpb, lds, stream);
  }
  if (cpw == 2) return launch_persist_cpw<MODE, 2>(pr, g, nw, tpb, lds, stream);
  if (cpw == 4) return launch_persist_cpw<MODE, 4>(pr, g, nw, tpb, lds, stream);
  return launch_persist_cpw<MODE, 7>(pr, g, nw, tpb, lds, stream);
}

bool dec_ok(int64_t t, int64_t k, const void* packed, const void* xq) {
  return dec_shape_ok(t, k, 0) && (reinterpret_cast<uintptr_t>(packed) % 16) == 0 &&
         (reinterpret_cast<uintptr_t>(xq) % 16) == 0;
}

hipError_t run_dec_int8(const uint8_t* packed, const float* gamma, const int8_t* xq,
                        const float* absmax, const int32_t* rowsum, int t, int n, int k, float* y,
                        int32_t* acc, const float* gamma2, uint16_t* h, hipStream_t stream) {
  DecGroup grp = {};
  grp.T = t;
  grp.p[0] = DecProblem{reinterpret_cast<const uint32_t*>(packed), gamma, xq, absmax, y, acc,
                        nullptr, nullptr, gamma2, h, n, k, 0, 0, rowsum};
  if (h == nullptr && t <= BL_GEMV_PERSIST_INT8_MAX_T && k <= BL_GEMV_PERSIST_INT8_MAX_K &&
      persist_ok(1, n, k)) {
    // one to four tokens over many tiles: the persistent kernel (the int8
    // rows staged once per block)
    DecProblem pr = grp.p[0];
    pr.ldy = n;
    return run_persist<kInt8>(pr, stream, t);
  }
  const int blocks = (n + 15) / 16;
  const DecShape sh = dec_shape(blocks, k, t);
  return run_dec<kInt8>(grp, 1, sh, dec_lds(t, k, 0, sh.rt), stream);
}

}  // namespace

int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    v = 256;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

hipError_t launch_linear_group(const bl_linear* probs, int count, int64_t t, int bf16,
                               hipStream_t stream) {
  const int rb = bf16 ? 2 : 4;   // bytes per raw activation
  // Fused, every block quantises the whole activation rows again: worth it
  // while that redundant work stays below a separate act-quant launch
  bool fused = count <= kMaxGroup;
  int64_t work = 0;
  for (int i = 0; fused && i < count; ++i) {
    fused = dec_shape_ok(t, probs[i].K, rb) &&
            (reinterpret_cast<uintptr_t>(probs[i].x) % 16) == 0 &&
            (reinterpret_cast<uintptr_t>(probs[i].packed) % 16) == 0;
    work += (probs[i].N + 15) / 16 * probs[i].K;
  }
  if (count == 1 && fused && persist_ok(t, probs[0].N, probs[0].K)) {
    // one token over many tiles: the persistent kernel quantises once per block
    const bl_linear& q = probs[0];
    const DecProblem pr{reinterpret_cast<const uint32_t*>(q.packed), q.gamma, q.x, nullptr, q.y,
                        q.acc, q.xq, q.absmax, nullptr, nullptr, (int)q.N, (int)q.K, 0,
                        (int)q.N, nullptr};
    return bf16 ? run_persist<kBf16>(pr, stream) : run_persist<kF32>(pr, stream);
  }
  if (!fuse_work_ok(t, work)) fused = false;
  if (!fused) {  // act-quant then forward (kernel chosen by T), problem by problem
    for (int i = 0; i < count; ++i) {
      const bl_linear& q = probs[i];
      hipError_t e = launch_quant(q.x, bf16, t, q.K, q.xq, q.absmax, nullptr, stream);
      if (e != hipSuccess) return e;
      e = auto_algo(t, q.N, q.K) == BL_ALGO_GEMV
              ? launch_gemv(q.packed, q.gamma, q.xq, q.absmax, nullptr, t, q.N, q.K, q.y, q.acc,
                            stream)
              : launch_gemm(q.packed, q.gamma, q.xq, q.absmax, nullptr, t, q.N, q.K, q.y, q.acc,
                            stream);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  // one block shape for the group: sized for the widest K and all 16-row tiles
  int64_t tiles = 0, kmax = 0;
  for (int i = 0; i < count; ++i) {
    tiles += (probs[i].N + 15) / 16;
    kmax = probs[i].K > kmax ? probs[i].K : kmax;
  }
  const DecShape sh = dec_shape(tiles, kmax, t);
  const size_t lds = dec_lds(t, kmax, rb, sh.rt);
  // The grid is (most blocks of a problem) x (problems), so blocks past a
  // narrower problem's rows only launch and exit, and they delay the
  // dispatch of the problems after them.  When the problems' block counts
  // differ, each wider one is cut into row ranges of about the narrowest
  // one's count (problems of their own, writing rows row0 .. of y with y's
  // full row stride) while at most kMaxGroup of them result.
  const int64_t brows = 16 * sh.rt;                 // weight rows per block
  int64_t bmin = INT64_MAX;
  for (int i = 0; i < count; ++i) {
    const int64_t b = (probs[i].N + brows - 1) / brows;
    bmin = b < bmin ? b : bmin;
  }
  int pieces = 0;
  for (int i = 0; i < count; ++i) pieces += (int)(((probs[i].N + brows - 1) / brows + bmin - 1) / bmin);
  const bool cut = pieces <= kMaxGroup;
  DecGroup grp = {};
  grp.T = (int)t;
  int np = 0;
  for (int i = 0; i < count; ++i) {
    const bl_linear& q = probs[i];
    const int64_t step = cut ? bmin * brows : q.N;  // rows per piece
    for (int64_t row0 = 0; row0 < q.N; row0 += step) {
      const int64_t rows = q.N - row0 < step ? q.N - row0 : step;
      const bool head = row0 == 0;                 // writes the int8 activations and absmax
      grp.p[np] = DecProblem{reinterpret_cast<const uint32_t*>(q.packed) + row0 * (q.K / 16),
                             q.gamma, q.x, nullptr, q.y + row0,
                             q.acc ? q.acc + row0 : nullptr, head ? q.xq : nullptr,
                             head ? q.absmax : nullptr, nullptr, nullptr, (int)rows, (int)q.K, 0,
                             (int)q.N, nullptr};
      ++np;
    }
  }
  return bf16 ? run_dec<kBf16>(grp, np, sh, lds, stream)
              : run_dec<kF32>(grp, np, sh, lds, stream);
}

namespace {

// The int8-input decode kernels, plain (y) or gated (gamma2 and h given).
hipError_t gemv_any(const uint8_t* packed, const float* gamma, const int8_t* xq,
                    const float* absmax, const int32_t* rowsum, int64_t t, int64_t n, int64_t k,
                    float* y, int32_t* acc, const float* gamma2, uint16_t* h,
                    hipStream_t stream) {
  if (dec_ok(t, k, packed, xq))
    return run_dec_int8(packed, gamma, xq, absmax, rowsum, (int)t, (int)n, (int)k, y, acc, gamma2,
                        h, stream);
  const bool vec4 = (k % 64) == 0 && (reinterpret_cast<uintptr_t>(packed) % 16) == 0 &&
                    (reinterpret_cast<uintptr_t>(xq) % 16) == 0;
  for (int64_t t0 = 0; t0 < t; t0 += kGemvTokens) {
    const int tc = (int)(t - t0 < kGemvTokens ? t - t0 : kGemvTokens);
    const int8_t* xs = xq + t0 * k;
    const int32_t* rs = rowsum ? rowsum + t0 : nullptr;
    float* ys = y ? y + t0 * n : nullptr;
    int32_t* as = acc ? acc + t0 * n : nullptr;
    uint16_t* hs = h ? h + t0 * (n / 2) : nullptr;
    if (vec4)
      run_tokens<4>(packed, gamma, xs, absmax + t0, rs, tc, (int)n, (int)k, ys, as, gamma2, hs,
                    stream);
    else
      run_tokens<1>(packed, gamma, xs, absmax + t0, rs, tc, (int)n, (int)k, ys, as, gamma2, hs,
                    stream);
  }
  return hipGetLastError();
}

}  // namespace

int auto_algo(int64_t t, int64_t n, int64_t k) {
  // The token count up to which the decode kernels beat the tiled MFMA
  // kernel (with its own tile choice and K split) depends on the matrix,
  // measured with weights rotated cold (decode / tiled, us):
  //  - up to 2 MB of packed weights, T = 64: 2560 -> 2560 9.1 / 11.3,
  //    2560 -> 640 9.0 / 10.5; at T = 96 the tiled kernel wins (14.9 / 11.9);
  //  - up to 16 MB, T = 32: 2560 -> 6912 8.6 / 11.9, 6912 -> 2560 11.6 / 12.1,
  //    3200 -> 8640 13.5 / 13.7, 8640 -> 3200 11.3 / 13.7; at T = 48 or 64
  //    the tiled kernel wins or ties (12.7 / 12.3, 14.7 / 13.2, 21.7 / 13.9,
  //    14.9 / 14.8);
  //  - larger (the 70B-class 58.7 MB), T = 6: 8192 -> 28672 23.3 / 25.5,
  //    28672 -> 8192 25.4 / 28.2; at T = 8 26.3 / 25.5 and 27.6 / 28.2, at
  //    T = 12 the tiled kernel wins on both (33.5 / 26.0, 34.1 / 29.2): past
  //    the decode kernel's LDS staging the 64-token kernel streams a large
  //    matrix slowly.
  const int64_t wbytes = n * (k / 4);
  const int64_t tmax = wbytes <= (int64_t(2) << 20) ? kGemvMaxTokens
                       : wbytes <= (int64_t(16) << 20) ? 32 : 6;
  return t <= tmax ? BL_ALGO_GEMV : BL_ALGO_GEMM;
}

hipError_t launch_gemv(const uint8_t* packed, const float* gamma, const int8_t* xq,
                       const float* absmax, const int32_t* rowsum, int64_t t, int64_t n,
                       int64_t k, float* y, int32_t* acc, hipStream_t stream) {
  return gemv_any(packed, gamma, xq, absmax, rowsum, t, n, k, y, acc, nullptr, nullptr, stream);
}

hipError_t launch_gemv_gated(const uint8_t* packed, const float* gamma_gate,
                             const float* gamma_up, const int8_t* xq, const float* absmax,
                             int64_t t, int64_t n, int64_t k, uint16_t* h, int32_t* acc,
                             hipStream_t stream) {
  return gemv_any(packed, gamma_gate, xq, absmax, nullptr, t, n, k, nullptr, acc, gamma_up, h,
                  stream);
}

hipError_t launch_gated(const void* x, int bf16, const uint8_t* packed, const float* gamma_gate,
                        const float* gamma_up, int64_t t, int64_t n, int64_t k, uint16_t* h,
                        int8_t* xq, float* absmax, int32_t* acc, hipStream_t stream) {
  const int rb = bf16 ? 2 : 4;
  const int64_t blocks = (n + 15) / 16;
  // one launch for decode shapes (the same rule as a grouped call of one problem)
  if (dec_shape_ok(t, k, rb) && (reinterpret_cast<uintptr_t>(x) % 16) == 0 &&
      (reinterpret_cast<uintptr_t>(packed) % 16) == 0 && fuse_work_ok(t, blocks * k)) {
    DecGroup grp = {};
    grp.T = (int)t;
    grp.p[0] = DecProblem{reinterpret_cast<const uint32_t*>(packed), gamma_gate, x, nullptr,
                          nullptr, acc, xq, absmax, gamma_up, h, (int)n, (int)k, 0, (int)n,
                          nullptr};
    const DecShape sh = dec_shape(blocks, k, t);
    const size_t lds = dec_lds(t, k, rb, sh.rt);
    return bf16 ? run_dec<kBf16>(grp, 1, sh, lds, stream)
                : run_dec<kF32>(grp, 1, sh, lds, stream);
  }
  hipError_t e = launch_quant(x, bf16, t, k, xq, absmax, nullptr, stream);
  if (e != hipSuccess) return e;
  return auto_algo(t, n, k) == BL_ALGO_GEMV
             ? launch_gemv_gated(packed, gamma_gate, gamma_up, xq, absmax, t, n, k, h, acc, stream)
             : launch_gemm_gated(packed, gamma_gate, gamma_up, xq, absmax, t, n, k, h, acc, stream);
}

}  // namespace bl
