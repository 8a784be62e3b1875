// Steps A2 + A3 for many tokens (prefill): a dense int8 contraction on the
// matrix cores, rescaled in the epilogue.
//
// The 2B4T report (section 5.1) keeps four ternary weights per byte in HBM,
// moves them on chip, unpacks them and multiplies with 8-bit activations.
// Here the int8 activations go through LDS (they are reused by every wave of
// the block), while the packed weights go straight from memory into
// registers: a lane loads 16 bytes (four packed words, 64 weights of one
// output row) per K step and expands them in registers,
//   codes = (word >> 2j) & 0x03030303,  t = byte-permute({-1,0,+1}, codes),
// two or three VALU operations per four weights, into MFMA B operands.
//
// v_mfma_i32_32x32x32_i8: A = 32 tokens x 32 k (from LDS), B = 32 k x 32
// output rows.  Within one MFMA the pairing of k with (lane half, byte) is
// free as long as A and B agree; this kernel gives lane half h of K-step s the
// 16 k of packed word 4h + s (relative to the 128-wide K tile), so the four
// words a lane needs over a K tile are contiguous in memory.
//
// Block: 2 x 2 waves, each owning WMF x WNF tiles of 32 x 32 outputs; K in
// steps of 128 with the activation tile double-buffered in LDS and the next
// tile's loads in flight during the current tile's MFMAs.  Tiles are ordered
// so that consecutive tiles of one XCD share activation rows in its L2.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "bl_internal.h"

namespace bl {
namespace {

constexpr int kThreads = 256;
constexpr int BK = 128;
constexpr int kLd = BK + 16;                  // LDS row stride (bytes): spreads banks
constexpr uint32_t kTernTable = 0x000100FFu;  // bytes {0xFF, 0x00, 0x01, 0x00}

__device__ __forceinline__ uint32_t signed_codes(uint32_t word, int j) {
  return __builtin_amdgcn_perm(kTernTable, kTernTable, codes_of(word, j));
}

// One-bit weights (bit u = 1 for +1, 0 for -1): bits j of the four bytes of a
// word are four consecutive k, taken as bytes u in {0, 1}; with t = 2u - 1,
// sum t*q = 2 * sum u*q - sum q.
__device__ __forceinline__ uint32_t bits_of(uint32_t word, int j) {
  return (word >> j) & 0x01010101u;
}

template <int WMF, int WNF>
__global__ __launch_bounds__(kThreads) void k_gemm(const uint32_t* __restrict__ packed,
                                                   const float* __restrict__ gamma,
                                                   const int8_t* __restrict__ xq,
                                                   const float* __restrict__ absmax, int T,
                                                   int N, int K, float* __restrict__ y,
                                                   int32_t* __restrict__ acc_out) {
  constexpr int BM = 2 * 32 * WMF, BN = 2 * 32 * WNF;
  constexpr int kAVec = BM * BK / 16 / kThreads;   // 16-byte A vectors per thread per tile
  extern __shared__ __align__(16) unsigned char smem[];
  int8_t* As = reinterpret_cast<int8_t*>(smem);    // [2][BM][kLd]
  float* scale = reinterpret_cast<float*>(smem + 2 * BM * kLd);  // [BM]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int K16 = K >> 4;

  // XCD-aware tile order: block b runs on XCD b % 8; give each XCD a
  // contiguous, M-major range of tiles.
  const int ntn = (N + BN - 1) / BN, ntm = (T + BM - 1) / BM;
  const int tiles = ntn * ntm;
  int tile = blockIdx.x;
  if (tiles >= 8 && (tiles % 8) == 0) tile = (blockIdx.x % 8) * (tiles / 8) + blockIdx.x / 8;
  const int m0 = (tile / ntn) * BM, n0 = (tile % ntn) * BN;

  // per-token output scale, once per block
  {
    const float g = gamma[0];
    for (int r = tid; r < BM; r += kThreads) {
      const int tok = m0 + r;
      scale[r] = tok < T ? out_scale(g, absmax[tok]) : 0.0f;
    }
  }

  // activation tile loader: thread handles kAVec 16-byte vectors
  auto load_a = [&](int k0, uint4 (&v)[kAVec]) {
#pragma unroll
    for (int u = 0; u < kAVec; ++u) {
      const int id = tid + u * kThreads;
      const int row = id / (BK / 16), c16 = id % (BK / 16);
      const int tok = m0 + row, kk = k0 + c16 * 16;
      v[u] = (tok < T && kk < K) ? *reinterpret_cast<const uint4*>(xq + (int64_t)tok * K + kk)
                                 : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_a = [&](int buf, const uint4 (&v)[kAVec]) {
#pragma unroll
    for (int u = 0; u < kAVec; ++u) {
      const int id = tid + u * kThreads;
      const int row = id / (BK / 16), c16 = id % (BK / 16);
      *reinterpret_cast<uint4*>(As + (buf * BM + row) * kLd + c16 * 16) = v[u];
    }
  };
  // weight words: lane (row l%32 of fragment j, half h = l/32) loads words
  // 4h .. 4h+3 of the K tile; rows past N read row N-1 (outputs discarded)
  const uint32_t* brow[WNF];
#pragma unroll
  for (int j = 0; j < WNF; ++j) {
    int n = n0 + wn * 32 * WNF + j * 32 + (lane & 31);
    n = n < N ? n : N - 1;
    brow[j] = packed + (int64_t)n * K16 + 4 * (lane >> 5);
  }
  auto load_b = [&](int k0, uint4 (&w)[WNF]) {
    const int wi = k0 >> 4;
#pragma unroll
    for (int j = 0; j < WNF; ++j) {
      // words wi+4h .. wi+4h+3 exist when K16 - wi >= 8; a K tail (K % 128)
      // reads word by word and zero-fills (the activations there are zero)
      if ((K16 & 3) == 0 && wi + 8 <= K16) {      // 16-byte aligned and in range
        w[j] = *reinterpret_cast<const uint4*>(brow[j] + wi);
      } else {
        const int h4 = 4 * (lane >> 5);
        uint32_t t[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) t[s] = (wi + h4 + s < K16) ? brow[j][wi + s] : 0u;
        w[j] = make_uint4(t[0], t[1], t[2], t[3]);
      }
    }
  };

  v16i acc[WMF][WNF];
#pragma unroll
  for (int i = 0; i < WMF; ++i)
#pragma unroll
    for (int j = 0; j < WNF; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;

  uint4 av[kAVec];
  uint4 bw[WNF], bw_next[WNF];
  load_a(0, av);
  load_b(0, bw);
  store_a(0, av);
  __syncthreads();

  const int ntiles_k = (K + BK - 1) / BK;
  for (int kt = 0; kt < ntiles_k; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < ntiles_k;
    // next tile's loads: activations first (waited on before the barrier),
    // then weights (consumed one iteration later)
    if (more) {
      load_a((kt + 1) * BK, av);
      load_b((kt + 1) * BK, bw_next);
    }
    const int8_t* At = As + (cur * BM + wm * 32 * WMF + (lane & 31)) * kLd + 64 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v4i a[WMF], b[WNF];
#pragma unroll
      for (int i = 0; i < WMF; ++i) {
        const uint4 t = *reinterpret_cast<const uint4*>(At + i * 32 * kLd + 16 * s);
        a[i] = v4i{(int)t.x, (int)t.y, (int)t.z, (int)t.w};
      }
#pragma unroll
      for (int j = 0; j < WNF; ++j) {
        const uint32_t w = s == 0 ? bw[j].x : s == 1 ? bw[j].y : s == 2 ? bw[j].z : bw[j].w;
        b[j] = v4i{(int)signed_codes(w, 0), (int)signed_codes(w, 1), (int)signed_codes(w, 2),
                   (int)signed_codes(w, 3)};
      }
#pragma unroll
      for (int i = 0; i < WMF; ++i)
#pragma unroll
        for (int j = 0; j < WNF; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      store_a(cur ^ 1, av);
#pragma unroll
      for (int j = 0; j < WNF; ++j) bw[j] = bw_next[j];
    }
    __syncthreads();
  }

  // epilogue: lane holds column (l % 32) of each fragment and rows
  // 8*(v/4) + 4*(l/32) + v%4; a register across the wave stores 32
  // consecutive outputs of two tokens
#pragma unroll
  for (int i = 0; i < WMF; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = wm * 32 * WMF + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
      const int tok = m0 + r;
      if (tok >= T) continue;
      const float sc = scale[r];
#pragma unroll
      for (int j = 0; j < WNF; ++j) {
        const int n = n0 + wn * 32 * WNF + j * 32 + (lane & 31);
        if (n >= N) continue;
        const int64_t o = (int64_t)tok * N + n;
        const int s = acc[i][j][v];
        if (acc_out) acc_out[o] = s;
        y[o] = (float)s * sc;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// LDS-direct variant (K % 128 == 0): both operands move global -> LDS with
// global_load_lds_dwordx4 (no VGPR staging), double-buffered, one barrier per
// 128-wide K step.  The instruction writes 64 lanes x 16 bytes contiguously,
// so the layout is chosen through the source addresses:
//   activations: 1 KiB = 8 rows x 128 bytes; row r's 16-byte slot p holds
//     logical slot p ^ ((r >> 1) & 7), spreading one MFMA read (32 rows, same
//     column) over the banks;
//   packed weights: 1 KiB = 32 rows x 32 bytes (8 words = 128 k), row-major.
// Each wave reads its four weight words per fragment with one 16-byte LDS
// read.  Two-bit weights go to the MFMA as their codes c = t + 1 in {0, 1, 2}
// (one or two VALU operations per four weights, no byte-permute), so the
// contraction yields sum c*q = sum t*q + sum q; each wave sums the q of the
// activation chunks it loaded itself (one LDS read and four dot4 operations
// per 1 KiB chunk and K step), and the epilogue subtracts each token's total
// over the block's K range (one-bit weights likewise go in as their bits u,
// and the epilogue forms 2 * sum u*q - sum q).  All of it is integer
// arithmetic: the result is the same exact int32 sum.  (Measured against the
// byte-permute expansion: T = 2048 prefill and 70B T = 256 4-8% faster.)
// s_waitcnt vmcnt(N) lgkmcnt(0)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0070 | (N & 15) | ((N >> 4) << 14));
}

#ifndef BL_GEMM_GROUP_M
#define BL_GEMM_GROUP_M 4   // row blocks per group of the tile order
#endif
#ifndef BL_GEMM_BREG
#define BL_GEMM_BREG 1      // two-bit weights of one-wave-row tiles straight into registers
#endif

// The exact sum from the contraction of the weight codes and the token's sum
// of q: two-bit codes c = t + 1 give sum t*q = acc - sum q, one-bit codes
// u = (t + 1) / 2 give sum t*q = 2 acc - sum q.
template <int WBITS>
__device__ __forceinline__ int exact_sum(int acc, int qsum) {
  return (WBITS == 2 ? acc : 2 * acc) - qsum;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* glb_ptr_t;

// 64 lanes x 16 bytes of zeros: the activation source of K-step slots past K
__device__ __align__(16) int8_t kZeroPage[1024];

// Each stage is its own static LDS object and every step below names its
// stages at compile time, so the compiler can tell that the loads landing in
// one stage do not alias reads of another and does not drain every
// outstanding load before each LDS read (one array indexed by stage is not
// enough for that).
//
// WBITS = 1: one-bit weights (K / 8 bytes per row; bit 8i + j of word g is
// k = 32g + 4j + i).  A K step then holds 4 words per row (16 bytes), step s
// and lane half h take word s, bits 4h .. 4h + 3 of each byte: k = 32s + 16h +
// [0, 16), which is 16-byte activation slot 2s + h.
//
// GATED: the weight rows come in (gate, up) pairs, 2i and 2i + 1, which sit in
// neighbouring lanes of a fragment; the even lane takes its neighbour's sum
// and writes the bfloat16 gated ReLU^2 of output i to h (y is not used).
// RS: each token's sum of q comes from rowsum[] (subtracted by the first K
// part only) instead of being summed from the activation tiles in the loop.
// TAIL: K % 128 == 64, so the last K step holds 64 k: its activation slots
// past K are read from a page of zeros and its weight loads past the row end
// reload the step's first half (multiplied by those zeros).  With K in parts
// the half step falls in the last part.
template <int WAVES, int WAVES_M, int WMF, int WNF, int STAGES, bool SPLIT, bool GATED,
          int WBITS = 2, bool RS = false, bool TAIL = false>
__global__ __launch_bounds__(WAVES * 64) void k_gemm_lds(const uint32_t* __restrict__ packed,
                                                         const float* __restrict__ gamma,
                                                         const int8_t* __restrict__ xq,
                                                         const float* __restrict__ absmax,
                                                         int T, int N, int K,
                                                         float* __restrict__ y,
                                                         int32_t* __restrict__ acc_out,
                                                         int ksteps, int splits,
                                                         const float* __restrict__ gamma2,
                                                         uint16_t* __restrict__ h_out,
                                                         const int32_t* __restrict__ rowsum) {
  static_assert(STAGES >= 2 && STAGES <= 4, "two to four stages");
  static_assert(!(RS && (GATED || WBITS != 2)), "rowsum: plain two-bit kernels only");
  static_assert(!(SPLIT && GATED), "the gated epilogue needs whole sums");
  static_assert(!(TAIL && (GATED || WBITS != 2)), "a half last K step: plain two-bit kernels");
  constexpr int NT = WAVES * 64;
  constexpr int WAVES_N = WAVES / WAVES_M;
  constexpr int BM = WAVES_M * 32 * WMF, BN = WAVES_N * 32 * WNF;
  static_assert(WBITS == 1 || WBITS == 2, "one- or two-bit weights");
  constexpr int kBRow = BK * WBITS / 8;                    // packed bytes per row per K step
  constexpr int kABuf = BM * BK, kBBuf = BN * kBRow;       // bytes per stage
  // 1 KiB loads per stage: kATot of the activation tile, kBTot of the
  // weights, shared out over the waves; where they do not divide evenly the
  // last waves load the tile's last chunk again (the same bytes to the same
  // LDS place), so every wave issues the same count
  constexpr int kATot = BM / 8, kBTot = kBBuf / 1024;
  constexpr int kAChunks = (kATot + WAVES - 1) / WAVES, kBChunks = (kBTot + WAVES - 1) / WAVES;
  static_assert(kBBuf % 1024 == 0, "weight tile in whole 1 KiB chunks");
  __shared__ __align__(16) unsigned char A0[kABuf], A1[kABuf];
  __shared__ __align__(16) unsigned char A2[STAGES > 2 ? kABuf : 16];
  __shared__ __align__(16) unsigned char A3[STAGES > 3 ? kABuf : 16];
  // Two-bit weights of a tile with one row of waves skip LDS: each weight
  // fragment is then read by one wave only, so each lane loads its own 16
  // bytes per fragment and step into registers, STAGES - 1 steps ahead (the
  // DMA write and the read of the weight tile leave the LDS traffic; T = 2048,
  // 2560 -> 6912: 43.9 -> 41.6-42.1 us; 70B T = 256, 8192 -> 28672: 65.2-66.2
  // -> 62.6-63.0 us).  With two rows of waves each fragment would be loaded
  // twice, and that measured slower (6912 -> 2560 on 64 x 320 tiles: 47.1 ->
  // 58.1 us).
  constexpr bool kBReg = BL_GEMM_BREG != 0 && WBITS == 2 && WAVES_M == 1;
  __shared__ __align__(16) unsigned char B0[kBReg ? 16 : kBBuf], B1[kBReg ? 16 : kBBuf];
  __shared__ __align__(16) unsigned char B2[STAGES > 2 && !kBReg ? kBBuf : 16];
  __shared__ __align__(16) unsigned char B3[STAGES > 3 && !kBReg ? kBBuf : 16];
  __shared__ float scale[BM];
  __shared__ double gm_gate[GATED ? BM : 1], gm_up[GATED ? BM : 1];   // gamma * m, binary64
  __shared__ int rsum[BM];   // each token's sum of q over the block's K range
  auto abuf = [&](auto st) -> unsigned char* {
    constexpr int S = decltype(st)::value;
    if constexpr (S == 0) return A0;
    else if constexpr (S == 1) return A1;
    else if constexpr (S == 2) return A2;
    else return A3;
  };
  auto bbuf = [&](auto st) -> unsigned char* {
    constexpr int S = decltype(st)::value;
    if constexpr (S == 0) return B0;
    else if constexpr (S == 1) return B1;
    else if constexpr (S == 2) return B2;
    else return B3;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int KW = K >> (WBITS == 2 ? 4 : 5);   // packed words per row

  const int ntn = (N + BN - 1) / BN, ntm = (T + BM - 1) / BM;
  const int tiles = ntn * ntm;
  // work item = (K part, tile); items next to each other share a K part, so
  // the blocks that run together share activation rows and weight columns
  const int items = SPLIT ? tiles * splits : tiles;
  int item = blockIdx.x;
  if (items >= 8 && (items % 8) == 0) item = (blockIdx.x % 8) * (items / 8) + blockIdx.x / 8;
  const int part = SPLIT ? item / tiles : 0, tile = item - part * tiles;
  // grouped order: BL_GEMM_GROUP_M row blocks at a time, down the rows first,
  // so that the contiguous range of tiles one XCD runs covers a squarer block
  // of the output (fewer distinct operand tiles through its L2)
  const int in_group = BL_GEMM_GROUP_M * ntn;
  const int gid = tile / in_group, first_m = gid * BL_GEMM_GROUP_M;
  const int gsize = min(ntm - first_m, BL_GEMM_GROUP_M);
  const int r_in = tile - gid * in_group;
  const int m0 = (first_m + r_in % gsize) * BM, n0 = (r_in / gsize) * BN;
  const uint32_t kbase = (uint32_t)part * (uint32_t)ksteps * BK;   // first k of this part

  // per-token output scale first: its loads retire before the pipeline starts
  {
    const float g = gamma[0];
    if constexpr (GATED) {
      const float g2 = gamma2[0];
      for (int r = tid; r < BM; r += NT) {
        const int tok = m0 + r;
        const float a = tok < T ? absmax[tok] : 0.0f;
        gm_gate[r] = gamma_m(g, a);
        gm_up[r] = gamma_m(g2, a);
      }
    } else {
      for (int r = tid; r < BM; r += NT) {
        const int tok = m0 + r;
        scale[r] = tok < T ? out_scale(g, absmax[tok]) : 0.0f;
        if constexpr (RS) rsum[r] = tok < T && part == 0 ? rowsum[tok] : 0;
      }
    }
  }

  // 32-bit offsets from the uniform bases (the host keeps T*K and N*K/16
  // below 2^31), so each load is a scalar base plus one VGPR offset
  uint32_t aoff[kAChunks], aslot[kAChunks];
#pragma unroll
  for (int i = 0; i < kAChunks; ++i) {
    const int c = min(wave * kAChunks + i, kATot - 1);
    const int r = 8 * c + (lane >> 3);
    const int slot = (lane & 7) ^ ((r >> 1) & 7);
    int tok = m0 + r;
    tok = tok < T ? tok : T - 1;
    aoff[i] = (uint32_t)tok * (uint32_t)K + 16u * slot;
    aslot[i] = 16u * slot;
  }
  uint32_t boff[kBChunks];
#pragma unroll
  for (int i = 0; i < kBChunks; ++i) {
    const int c = min(wave * kBChunks + i, kBTot - 1);
    if constexpr (WBITS == 2) {   // 1 KiB = 32 rows x 32 bytes
      int n = n0 + 32 * c + (lane >> 1);
      n = n < N ? n : N - 1;
      boff[i] = (uint32_t)n * (uint32_t)KW + 4u * (lane & 1);
    } else {                      // 1 KiB = 64 rows x 16 bytes
      int n = n0 + 64 * c + lane;
      n = n < N ? n : N - 1;
      boff[i] = (uint32_t)n * (uint32_t)KW;
    }
  }
  // register weights: lane (m, h) of fragment j takes row wn*32*WNF + 32j + m,
  // bytes 16h .. 16h + 15 of the step's 32
  uint32_t roff[kBReg ? WNF : 1];
  if constexpr (kBReg) {
#pragma unroll
    for (int j = 0; j < WNF; ++j) {
      int n = n0 + wn * 32 * WNF + 32 * j + (lane & 31);
      n = n < N ? n : N - 1;
      roff[j] = (uint32_t)n * (uint32_t)KW + 4u * (lane >> 5);
    }
  }
  uint4 breg[kBReg ? STAGES : 1][kBReg ? WNF : 1];
  const uint32_t h_of_lane = (uint32_t)lane >> 5;
  auto issue = [&](int kt, auto stage_c) {
    constexpr int S = decltype(stage_c)::value;
    unsigned char* As = abuf(stage_c);
    const uint32_t k0 = kbase + (uint32_t)kt * BK;
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      const int8_t* src = xq + (aoff[i] + k0);
      if constexpr (TAIL) src = k0 + aslot[i] < (uint32_t)K ? src : kZeroPage + 16 * lane;
      __builtin_amdgcn_global_load_lds((glb_ptr_t)src,
                                       (lds_ptr_t)(As + min(wave * kAChunks + i, kATot - 1) * 1024),
                                       16, 0, 0);
    }
    if constexpr (kBReg) {
      // the step's second half (h = 1) past the row end: the first half again
      const uint32_t back = TAIL && k0 + 64u * h_of_lane >= (uint32_t)K ? 4u : 0u;
#pragma unroll
      for (int j = 0; j < WNF; ++j)
        breg[S][j] = *reinterpret_cast<const uint4*>(packed + (roff[j] + (k0 >> 4) - back));
    } else {
      unsigned char* Bs = bbuf(stage_c);
      const uint32_t back = TAIL && k0 + 64u * (lane & 1) >= (uint32_t)K ? 4u : 0u;
#pragma unroll
      for (int i = 0; i < kBChunks; ++i)
        __builtin_amdgcn_global_load_lds((glb_ptr_t)(packed + (boff[i] + (k0 >> (WBITS == 2 ? 4 : 5)) - back)),
                                         (lds_ptr_t)(Bs + min(wave * kBChunks + i, kBTot - 1) * 1024),
                                         16, 0, 0);
    }
  };

  v16i acc[WMF][WNF];
#pragma unroll
  for (int i = 0; i < WMF; ++i)
#pragma unroll
    for (int j = 0; j < WNF; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0;

  int qpart[kAChunks];   // per lane: sum of q over its 16-byte pieces of chunk i
#pragma unroll
  for (int i = 0; i < kAChunks; ++i) qpart[i] = 0;

  const int nkall = (K + BK - 1) / BK;             // K steps, a half last one included
  const int nk = SPLIT ? min(ksteps, nkall - part * ksteps) : nkall;   // >= 1 (host)
  constexpr int kLoads = kAChunks + (kBReg ? WNF : kBChunks);   // this wave's loads per tile
  static_assert(kLoads * (STAGES - 2) < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0);                  // the scale loads
  // prologue: tiles 0 .. STAGES-2 (repeats of the last tile when K is short)
  issue(0, I0{});
  if constexpr (STAGES >= 3) issue(nk > 1 ? 1 : 0, I1{});
  if constexpr (STAGES == 4) issue(nk > 2 ? 2 : nk - 1, I2{});
  // tile 0 landed (the rest stays in flight) and the scale writes are done;
  // a fence-free barrier, as a fence would wait for every load
  wait_vm_lgkm0<kLoads * (STAGES - 2)>();
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);

  const int h = lane >> 5, m = lane & 31;
  const int aswz = (m >> 1) & 7;
  // With four stages the refill goes out after the step's MFMAs, not before
  // them: a wave issues in order, and while the CU's memory queue is full
  // the refill's loads are accepted only as data returns, holding the
  // step's LDS reads and MFMAs back; three stages in flight still cover
  // the loads' latency.  (70B T = 256, 28672 -> 8192 on 64 x 128 tiles:
  // 81.7-82.1 -> 79.4-79.6 us, 78.4 -> 72.5-73.6 with the row sums handed
  // in; on the other tile shapes within 2% either way, so they keep three
  // stages and the early refill.)
  constexpr bool kLateRefill = STAGES >= 4;
  // One K step on stage S; refill stage (S + STAGES - 1) % STAGES, which the
  // previous step finished reading, with tile kt + STAGES - 1.
  auto step = [&](auto stage_c, int kt) {
    constexpr int S = decltype(stage_c)::value;
    using R = std::integral_constant<int, (S + STAGES - 1) % STAGES>;
    // unconditional (no branch, so no join where the compiler would drain
    // every load): past the end it re-fetches the last tile into a stage that
    // is never read again
    auto refill = [&]() {
      issue(kt + STAGES - 1 < nk ? kt + STAGES - 1 : nk - 1, R{});
    };
    if constexpr (!kLateRefill) refill();
    const unsigned char* At = abuf(stage_c) + (wm * 32 * WMF + m) * BK;
    const unsigned char* Bt =
        bbuf(stage_c) + (wn * 32 * WNF + m) * kBRow + (WBITS == 2 ? 16 * h : 0);
    if constexpr (!RS) {
      // this wave's own activation chunks of the step (rows 8c .. 8c + 7,
      // 16 bytes per lane, slot order irrelevant to a sum): sum of q
#pragma unroll
      for (int i = 0; i < kAChunks; ++i) {
        const uint4 v = *reinterpret_cast<const uint4*>(
            abuf(stage_c) + min(wave * kAChunks + i, kATot - 1) * 1024 + 16 * lane);
        int p = qpart[i];
        p = __builtin_amdgcn_sdot4((int)v.x, 0x01010101, p, false);
        p = __builtin_amdgcn_sdot4((int)v.y, 0x01010101, p, false);
        p = __builtin_amdgcn_sdot4((int)v.z, 0x01010101, p, false);
        qpart[i] = __builtin_amdgcn_sdot4((int)v.w, 0x01010101, p, false);
      }
    }
    uint4 bw[WNF];
#pragma unroll
    for (int j = 0; j < WNF; ++j) {
      if constexpr (kBReg) bw[j] = breg[S][j];
      else bw[j] = *reinterpret_cast<const uint4*>(Bt + j * 32 * kBRow);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int off = 16 * ((WBITS == 2 ? 4 * h + s : 2 * s + h) ^ aswz);
      v4i a[WMF];
#pragma unroll
      for (int i = 0; i < WMF; ++i) {
        const uint4 t = *reinterpret_cast<const uint4*>(At + i * 32 * BK + off);
        a[i] = v4i{(int)t.x, (int)t.y, (int)t.z, (int)t.w};
      }
#pragma unroll
      for (int j = 0; j < WNF; ++j) {
        // expand one weight fragment right before its MFMAs (few live registers)
        const uint32_t w = s == 0 ? bw[j].x : s == 1 ? bw[j].y : s == 2 ? bw[j].z : bw[j].w;
        v4i b;
        if constexpr (WBITS == 2) {
          // codes c = t + 1 as they are: sum c * q = sum t * q + sum q
          b = v4i{(int)codes_of(w, 0), (int)codes_of(w, 1), (int)codes_of(w, 2),
                  (int)codes_of(w, 3)};
        } else {
          const uint32_t wh = w >> (4 * h);
          b = v4i{(int)bits_of(wh, 0), (int)bits_of(wh, 1), (int)bits_of(wh, 2),
                  (int)bits_of(wh, 3)};
        }
#pragma unroll
        for (int i = 0; i < WMF; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b, acc[i][j], 0, 0, 0);
      }
      // no scheduling fence between sub-steps: letting the compiler overlap
      // one sub-step's LDS reads with the previous one's MFMAs measured 1-4%
      // faster at the same register count
    }
    if constexpr (kLateRefill) refill();
    // Tile kt+1 must have landed: this wave's loads by the wait, everyone's
    // by the barrier.  A plain s_barrier, not __syncthreads(): the latter's
    // release fence would also wait for the refill issued above.  The only
    // LDS writes in the loop are these loads, which the wait covers.
    wait_vmem<kLoads * (STAGES - 2)>();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // whole stage cycles without conditionals (branch joins make the compiler
  // drain every outstanding load), then the remaining steps
  int kt = 0;
  for (; kt + STAGES <= nk; kt += STAGES) {
    step(I0{}, kt);
    step(I1{}, kt + 1);
    if constexpr (STAGES >= 3) step(I2{}, kt + 2);
    if constexpr (STAGES == 4) step(I3{}, kt + 3);
  }
  if (kt < nk) step(I0{}, kt);
  if constexpr (STAGES >= 3)
    if (kt + 1 < nk) step(I1{}, kt + 1);
  if constexpr (STAGES == 4)
    if (kt + 2 < nk) step(I2{}, kt + 2);
  wait_vmem<0>();   // no load may land in LDS after the block has finished
  if constexpr (!RS) {
    // eight lanes hold the pieces of one row of a chunk: their total is the
    // token's sum of q over this block's K range
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      int v = qpart[i];
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      v += __shfl_xor(v, 4);
      // a repeated chunk writes the same sums again
      if ((lane & 7) == 0) rsum[8 * min(wave * kAChunks + i, kATot - 1) + (lane >> 3)] = v;
    }
    lds_sync();
  }

  if constexpr (GATED) {
    const int half = N >> 1;
#pragma unroll
    for (int i = 0; i < WMF; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * 32 * WMF + i * 32 + (v >> 2) * 8 + h * 4 + (v & 3);
        const int tok = m0 + r;
        const double gg = gm_gate[r], gu = gm_up[r];
        const int qs = rsum[r];
#pragma unroll
        for (int j = 0; j < WNF; ++j) {
          const int n = n0 + wn * 32 * WNF + j * 32 + m;
          const int sv = exact_sum<WBITS>(acc[i][j][v], qs);
          // every lane takes part: lane l gets lane l ^ 1's sum
          const int other = __builtin_amdgcn_update_dpp(0, sv, 0xB1, 0xF, 0xF, false);
          if (tok >= T || n >= N) continue;
          const int64_t o = (int64_t)tok * N + n;
          if (acc_out) acc_out[o] = sv;
          if ((m & 1) == 0)
            h_out[(int64_t)tok * half + (n >> 1)] = gated_relu2_bf16(sv, other, gg, gu);
        }
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < WMF; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = wm * 32 * WMF + i * 32 + (v >> 2) * 8 + h * 4 + (v & 3);
      const int tok = m0 + r;
      if (tok >= T) continue;
      const float sc = scale[r];
      const int qs = rsum[r];
#pragma unroll
      for (int j = 0; j < WNF; ++j) {
        const int n = n0 + wn * 32 * WNF + j * 32 + m;
        if (n >= N) continue;
        const int64_t o = (int64_t)tok * N + n;
        const int sv = exact_sum<WBITS>(acc[i][j][v], qs);
        if constexpr (SPLIT) {
          // K split: exact int32 partial sums meet in y (zeroed beforehand,
          // read as int32 until the finishing pass rescales it in place)
          atomicAdd(reinterpret_cast<int*>(y) + o, sv);
        } else {
          if (acc_out) acc_out[o] = sv;
          y[o] = (float)sv * sc;
        }
      }
    }
  }
}

// K split, around the kernel above: y is cleared, receives the exact int32
// partial sums of every K part (integer addition, so the order of the atomic
// adds does not matter), and is then rescaled in place.
__global__ __launch_bounds__(256) void k_clear_i32(int* __restrict__ p, int64_t n) {
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0;
}

// one block per (row, 1024-column block)
__global__ __launch_bounds__(256) void k_split_finish(float* __restrict__ y,
                                                      int32_t* __restrict__ acc_out,
                                                      const float* __restrict__ gamma,
                                                      const float* __restrict__ absmax, int N,
                                                      int col_blocks) {
  const int t = blockIdx.x / col_blocks, cb = blockIdx.x - t * col_blocks;
  const float sc = out_scale(gamma[0], absmax[t]);
  const int64_t row = (int64_t)t * N;
  for (int c = cb * 1024 + threadIdx.x; c < min(N, cb * 1024 + 1024); c += 256) {
    const int v = reinterpret_cast<const int*>(y)[row + c];
    if (acc_out) acc_out[row + c] = v;
    y[row + c] = (float)v * sc;
  }
}

template <int WAVES, int WAVES_M, int WMF, int WNF, int STAGES, bool GATED = false, int WBITS = 2>
hipError_t run_lds(const uint8_t* packed, const float* gamma, const int8_t* xq,
                   const float* absmax, int64_t t, int64_t n, int64_t k, float* y, int32_t* acc,
                   hipStream_t stream, int splits = 1, int ksteps = 0,
                   const float* gamma2 = nullptr, uint16_t* h = nullptr,
                   const int32_t* rowsum = nullptr) {
  // K parts of ksteps 128-wide steps each (the last may be shorter); the
  // caller sizes them so that every part has at least one step
  if (splits == 1) ksteps = (int)(k / BK);
  constexpr int BM = WAVES_M * 32 * WMF, BN = (WAVES / WAVES_M) * 32 * WNF;
  const int64_t tiles = ((n + BN - 1) / BN) * ((t + BM - 1) / BM);
  // only the kernels a configuration uses are instantiated
  auto pick = [&]() {
    if constexpr (WBITS == 1)
      return k_gemm_lds<WAVES, WAVES_M, WMF, WNF, STAGES, false, false, 1>;
    else if constexpr (GATED)
      return k_gemm_lds<WAVES, WAVES_M, WMF, WNF, STAGES, false, true>;
    else if (k % BK != 0)   // K % 128 == 64 (host): a half last step
      return rowsum ? (splits > 1 ? k_gemm_lds<WAVES, WAVES_M, WMF, WNF, STAGES, true, false, 2, true, true>
                                  : k_gemm_lds<WAVES, WAVES_M, WMF, WNF, STAGES, false, false, 2, true, true>)
                    : (splits > 1 ? k_gemm_lds<WAVES, WAVES_M, WMF, WNF, STAGES, true, false, 2, false, true>
                                  : k_gemm_lds<WAVES, WAVES_M, WMF, WNF, STAGES, false, false, 2, false, true>);
    else if (rowsum)
      return splits > 1 ? k_gemm_lds<WAVES, WAVES_M, WMF, WNF, STAGES, true, false, 2, true>
                        : k_gemm_lds<WAVES, WAVES_M, WMF, WNF, STAGES, false, false, 2, true>;
    else
      return splits > 1 ? k_gemm_lds<WAVES, WAVES_M, WMF, WNF, STAGES, true, false>
                        : k_gemm_lds<WAVES, WAVES_M, WMF, WNF, STAGES, false, false>;
  };
  auto kern = pick();
  kern<<<dim3((unsigned)(tiles * splits)), WAVES * 64, 0, stream>>>(
      reinterpret_cast<const uint32_t*>(packed), gamma, xq, absmax, (int)t, (int)n, (int)k, y, acc,
      ksteps, splits, gamma2, h, rowsum);
  return hipGetLastError();
}

template <int WMF, int WNF>
hipError_t run(const uint8_t* packed, const float* gamma, const int8_t* xq, const float* absmax,
               int64_t t, int64_t n, int64_t k, float* y, int32_t* acc, hipStream_t stream) {
  constexpr int BM = 64 * WMF, BN = 64 * WNF;
  const int64_t tiles = ((n + BN - 1) / BN) * ((t + BM - 1) / BM);
  const size_t lds = 2 * (size_t)BM * kLd + BM * sizeof(float);
  auto kern = k_gemm<WMF, WNF>;
  // the LDS limit is raised once per device (setting it again is harmless,
  // so two threads racing here is fine)
  static std::atomic<uint64_t> lds_set{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? uint64_t(1) << dev : 0;
  if (bit == 0 || !(lds_set.load(std::memory_order_relaxed) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    lds_set.fetch_or(bit, std::memory_order_relaxed);
  }
  kern<<<dim3((unsigned)tiles), kThreads, lds, stream>>>(reinterpret_cast<const uint32_t*>(packed),
                                                         gamma, xq, absmax, (int)t, (int)n,
                                                         (int)k, y, acc);
  return hipGetLastError();
}

}  // namespace

#ifndef BL_GEMM_BIG_MIN_TILES
#define BL_GEMM_BIG_MIN_TILES 384   // K % 128 != 0: 256 x 128 tiles when at least this many exist
#endif
#ifndef BL_GEMM_WIDE_MIN_TILES
#define BL_GEMM_WIDE_MIN_TILES 160  // 128 x 512 tiles from this many on
#endif
#ifndef BL_GEMM_NARROW_MIN_TILES
#define BL_GEMM_NARROW_MIN_TILES 224  // 128 x 256 tiles from this many on (rows at least 90% used)
#endif
#ifndef BL_GEMM_M64_MIN_TILES
#define BL_GEMM_M64_MIN_TILES 256   // 64 x 256 tiles from this many on, else 64 x 128
#endif
#ifndef BL_GEMM_STAGES
#define BL_GEMM_STAGES 3            // LDS pipeline depth (tiles in flight + 1)
#endif
#ifndef BL_GEMM_SPLIT_ITEMS
#define BL_GEMM_SPLIT_ITEMS 256     // K split: (part, tile) items aimed for
#endif
#ifndef BL_GEMM_SPLIT_MIN_K
#define BL_GEMM_SPLIT_MIN_K 16384   // K split only for long rows ...
#endif
#ifndef BL_GEMM_SPLIT_MAX_TILES
#define BL_GEMM_SPLIT_MAX_TILES 128 // ... that make fewer than this many 64 x 128 tiles
#endif
#ifndef BL_GEMM_SPLIT64_WIDE_TILES
#define BL_GEMM_SPLIT64_WIDE_TILES 96   // any T: 64 x 128 tiles in K parts below this many ...
#endif
#ifndef BL_GEMM_SPLIT64_WIDE_STEPS
#define BL_GEMM_SPLIT64_WIDE_STEPS 32   // ... when the rows take at least this many 128-wide steps
#endif
#ifndef BL_GEMM_SPLIT64_MAX_TILES
#define BL_GEMM_SPLIT64_MAX_TILES 40    // up to 64 tokens: 64 x 128 tiles in K parts below this many
// (T = 64, 6912 -> 2560, 20 tiles: 23.9 -> 14.1 us; 2560 -> 6912, 54 tiles:
// 12.4 -> 16.5 us, the clearing and finishing launches costing more there)
#endif


namespace {

// Tile shape of the LDS-direct kernel for a problem, from measurements on
// MI355X over T in 160..8192 and the 2B / 70B-class shapes: the widest tiles
// that still give most CUs a block, 64-row tiles (several blocks per CU) when
// 128-row ones would leave CUs idle or rows unused, and a K split only for
// long K with very few tiles.
enum class Tiles { kWide, kNarrow, kM64W256, kM64W320, kM64W128, kSplit, kSplit64 };

Tiles choose_tiles(int64_t t, int64_t n, int64_t k, bool allow_split, bool allow_w128,
                   bool allow_w320 = false) {
  const int64_t m128 = (t + 127) / 128, m64 = (t + 63) / 64;
  const int64_t wide = m128 * ((n + 511) / 512), narrow = m128 * ((n + 255) / 256);
  const int64_t w256 = m64 * ((n + 255) / 256), w128 = m64 * ((n + 127) / 128);
  const bool rows_used = 10 * t >= 9 * 128 * m128;   // 128-row tiles at least 90% full
  const int64_t cus = device_cus();
  // 128-row tiles that would leave a second round less than a quarter full
  // take 64 x 256 tiles, several blocks of which share a CU in one round
  // (T = 2048, 3200 -> 8640: 272 tiles of 128 x 512, 83.5 us; 544 of
  // 128 x 256, 92.6 us; 1088 of 64 x 256, 71.1 us)
  const bool wide_spills = wide > cus && 4 * wide < 5 * cus;
  if (wide >= BL_GEMM_WIDE_MIN_TILES && !wide_spills) return Tiles::kWide;
  if (narrow >= BL_GEMM_NARROW_MIN_TILES && rows_used && !wide_spills) return Tiles::kNarrow;
  if (w256 >= BL_GEMM_M64_MIN_TILES || !allow_w128 || wide_spills) {
    // 64 x 256 tiles that would spill into a second round, where 64 x 320
    // tiles fill the CUs once (2048 x 6912 -> 2560: 320 against 256 tiles,
    // 48.5 -> 43.9 us; 128 x 160 tiles measured 46.0 us)
    const int64_t w320 = m64 * ((n + 319) / 320);
    if (allow_w320 && w256 > cus && 8 * w320 >= 7 * cus && w320 <= cus) return Tiles::kM64W320;
    return Tiles::kM64W256;
  }
  // a few tokens over few tiles: 64-row tiles, K in parts, so that the
  // launch has work for every CU
  if (allow_split && t <= 64 && w128 < BL_GEMM_SPLIT64_MAX_TILES && k / BK >= 8)
    return Tiles::kSplit64;
  // any T over few tiles of long rows: the same split (6912 -> 2560 at
  // T = 128 / 256, 40 / 80 tiles of 54 steps: 22.9 / 23.0 -> 18.0 / 21.6 us;
  // with rows of 20 steps, 2560 -> 6912, it did not pay at 54 tiles)
  if (allow_split && w128 < BL_GEMM_SPLIT64_WIDE_TILES && k / BK >= BL_GEMM_SPLIT64_WIDE_STEPS)
    return Tiles::kSplit64;
  if (allow_split && k >= BL_GEMM_SPLIT_MIN_K && w128 < BL_GEMM_SPLIT_MAX_TILES && k / BK >= 8)
    return Tiles::kSplit;
  return Tiles::kM64W128;
}

}  // namespace

hipError_t launch_gemm(const uint8_t* packed, const float* gamma, const int8_t* xq,
                       const float* absmax, const int32_t* rowsum, int64_t t, int64_t n,
                       int64_t k, float* y, int32_t* acc, hipStream_t stream) {
  // K % 128 == 64 takes the same kernels with a half last step
  const bool lds_ok = k % 64 == 0 && t * k < (int64_t(1) << 31) && n * (k / 16) < (int64_t(1) << 31);
  if (!lds_ok) {
    // K % 64 != 0 (or offsets beyond 32 bits): the register-staged kernel
    const int64_t big = ((n + 127) / 128) * ((t + 255) / 256);
    if (big >= BL_GEMM_BIG_MIN_TILES)
      return run<4, 2>(packed, gamma, xq, absmax, t, n, k, y, acc, stream);
    return run<2, 2>(packed, gamma, xq, absmax, t, n, k, y, acc, stream);
  }
  const Tiles choice = choose_tiles(t, n, k, t * n < (int64_t(1) << 31), true, true);
  switch (choice) {
    case Tiles::kWide:
      return run_lds<8, 1, 4, 2, BL_GEMM_STAGES>(packed, gamma, xq, absmax, t, n, k, y, acc, stream,
                                                 1, 0, nullptr, nullptr, rowsum);
    case Tiles::kNarrow:
      // eight waves of 128 x 32 (two per SIMD) rather than four of 128 x 64:
      // 70B T = 256, 8192 -> 28672 62.4-65.6 -> 58.9-60.2 us; T = 512,
      // 4096 -> 14336 37.7 -> 34.3 us; T = 2048, 320 -> 3500 16.8 -> 12.5 us
      // (two rows of four waves with the weights through LDS: 60.9 us)
      return run_lds<8, 1, 4, 1, BL_GEMM_STAGES>(packed, gamma, xq, absmax, t, n, k, y, acc, stream,
                                                 1, 0, nullptr, nullptr, rowsum);
    case Tiles::kM64W256:
      return run_lds<4, 1, 2, 2, BL_GEMM_STAGES>(packed, gamma, xq, absmax, t, n, k, y, acc, stream,
                                                 1, 0, nullptr, nullptr, rowsum);
    case Tiles::kM64W320:
      // ten waves of 32 x 64 (2 x 5; two or three per SIMD) rather than four
      // of 32 x 160: T = 2048, 6912 -> 2560 44.3 -> 43.2 us, 8192 -> 2560
      // 50.0 -> 49.0 us, T = 2000, 1024 -> 2500 15.5 -> 13.1 us
      return run_lds<10, 2, 1, 2, BL_GEMM_STAGES>(packed, gamma, xq, absmax, t, n, k, y, acc, stream,
                                                  1, 0, nullptr, nullptr, rowsum);
    case Tiles::kM64W128:
      // eight waves of 32 x 32 (two per SIMD) rather than four of 32 x 64:
      // 70B T = 256, 28672 -> 8192 78.6 -> 75.2 us; T = 64, 2560 -> 6912
      // 12.1 -> 10.7 us; T = 200, 8192 -> 4000 25.3 -> 23.2 us (the K split
      // keeps four waves: equal or 4% slower with eight)
      return run_lds<8, 2, 1, 1, 4>(packed, gamma, xq, absmax, t, n, k, y, acc, stream,
                                    1, 0, nullptr, nullptr, rowsum);
    case Tiles::kSplit:
    case Tiles::kSplit64: {
      // 128 x 512 (or, up to 64 tokens, 64 x 128) tiles, K in parts: y is
      // cleared, takes the exact int32 partial sums by atomics and is
      // rescaled in place
      const bool t64 = choice == Tiles::kSplit64;
      const int64_t nkt = (k + BK - 1) / BK;        // a half last step (K % 128 == 64) included
      const int64_t tl = t64 ? ((t + 63) / 64) * ((n + 127) / 128)
                             : ((t + 127) / 128) * ((n + 511) / 512);
      int64_t parts = (BL_GEMM_SPLIT_ITEMS + tl - 1) / tl;
      int64_t steps = (nkt + parts - 1) / parts;
      if (steps < 4) steps = 4;
      parts = (nkt + steps - 1) / steps;             // every part has at least one step
      const int64_t total = t * n;
      k_clear_i32<<<(unsigned)std::min<int64_t>((total + 255) / 256, 4096), 256, 0, stream>>>(
          reinterpret_cast<int*>(y), total);
      hipError_t e =
          t64 ? run_lds<4, 2, 1, 2, 4>(packed, gamma, xq, absmax, t, n, k, y, acc, stream,
                                       (int)parts, (int)steps, nullptr, nullptr, rowsum)
              : run_lds<8, 1, 4, 2, BL_GEMM_STAGES>(packed, gamma, xq, absmax, t, n, k, y, acc,
                                                    stream, (int)parts, (int)steps, nullptr,
                                                    nullptr, rowsum);
      if (e != hipSuccess) return e;
      const int col_blocks = (int)((n + 1023) / 1024);
      k_split_finish<<<(unsigned)(t * col_blocks), 256, 0, stream>>>(y, acc, gamma, absmax, (int)n,
                                                                     col_blocks);
      return hipGetLastError();
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_gated(const uint8_t* packed, const float* gamma_gate,
                             const float* gamma_up, const int8_t* xq, const float* absmax,
                             int64_t t, int64_t n, int64_t k, uint16_t* h, int32_t* acc,
                             hipStream_t stream) {
  // LDS-direct tiles only (no K split: the epilogue needs whole sums); other
  // shapes go to the decode kernel, which takes any T
  const bool lds_ok = k % BK == 0 && t * k < (int64_t(1) << 31) && n * (k / 16) < (int64_t(1) << 31);
  if (!lds_ok)
    return launch_gemv_gated(packed, gamma_gate, gamma_up, xq, absmax, t, n, k, h, acc, stream);
  switch (choose_tiles(t, n, k, false, true)) {
    case Tiles::kWide:
      return run_lds<8, 1, 4, 2, BL_GEMM_STAGES, true>(packed, gamma_gate, xq, absmax, t, n, k,
                                                       nullptr, acc, stream, 1, 0, gamma_up, h);
    case Tiles::kNarrow:
      // eight waves of 128 x 32 (T = 640, 2560 -> 2 x 6912: 65.7 -> 53.4 us)
      return run_lds<8, 1, 4, 1, BL_GEMM_STAGES, true>(packed, gamma_gate, xq, absmax, t, n, k,
                                                       nullptr, acc, stream, 1, 0, gamma_up, h);
    case Tiles::kM64W256:
      return run_lds<4, 1, 2, 2, BL_GEMM_STAGES, true>(packed, gamma_gate, xq, absmax, t, n, k,
                                                       nullptr, acc, stream, 1, 0, gamma_up, h);
    default:
      // eight waves of 32 x 32, as the plain kernel (act-quant + gated GEMM
      // on 2560 -> 2 x 6912: T = 128 16.9 -> 14.7 us, T = 256 22.3 -> 21.3)
      return run_lds<8, 2, 1, 1, BL_GEMM_STAGES, true>(packed, gamma_gate, xq, absmax, t, n, k,
                                                       nullptr, acc, stream, 1, 0, gamma_up, h);
  }
}

hipError_t launch_gemm_binary(const uint8_t* packed, const float* gamma, const int8_t* xq,
                              const float* absmax, int64_t t, int64_t n, int64_t k, float* y,
                              int32_t* acc, hipStream_t stream) {
  // the host keeps the kernel's 32-bit offsets in range (K % 128 == 0 by the
  // caller); one-bit rows give a 64 x 128 tile too few bytes per wave, so
  // 64 x 256 is the smallest tile here
  switch (choose_tiles(t, n, k, false, false)) {
    case Tiles::kWide:
      return run_lds<8, 1, 4, 2, BL_GEMM_STAGES, false, 1>(packed, gamma, xq, absmax, t, n, k, y,
                                                           acc, stream);
    case Tiles::kNarrow:
      return run_lds<4, 1, 4, 2, BL_GEMM_STAGES, false, 1>(packed, gamma, xq, absmax, t, n, k, y,
                                                           acc, stream);
    default:
      return run_lds<4, 1, 2, 2, BL_GEMM_STAGES, false, 1>(packed, gamma, xq, absmax, t, n, k, y,
                                                           acc, stream);
  }
}

}  // namespace bl
