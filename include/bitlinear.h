/*
 * bitlinear.h -- C ABI of the BitLinear (W1.58A8) forward on AMD Instinct
 * MI355X (gfx950).
 *
 * BitLinear replaces a bias-free torch.nn.Linear ("BitNet b1.58 2B4T
 * Technical Report", section 2, architecture; same section of the English
 * summary "BitNet b1.58 2B4T Technical Report | Summary").  Its forward has
 * four steps, and this library runs each of them in hand-written HIP kernels:
 *
 *   A0  absmean ternarisation of the latent weights to {-1, 0, +1} with one
 *       scale gamma per matrix, stored at 2 bits per weight
 *       ("BitNet解读", weight quantisation function, eq. (1)-(3);
 *        2B4T report section 5.1: four ternary values per 8-bit integer);
 *   A1  per-token absmax quantisation of the activations to int8
 *       ("BitNet解读", activation quantisation; 2B4T report section 2);
 *   A2  the ternary x int8 contraction into exact int32 sums
 *       ("BitNet解读", computational efficiency: +1 adds, -1 subtracts,
 *        0 skips);
 *   A3  the rescale of each sum by gamma times the activation scale
 *       (bitnet.cpp post on gitcode.csdn.net, section 1.1: a scale factor
 *        restores the range of the ternary weights).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Tensor pointers are DEVICE pointers into row-major buffers that the
 *   caller allocates and owns; outputs are written in place.  The library
 *   keeps no state between calls and never allocates device memory; its one
 *   piece of device memory is the fixed 2 KiB array that
 *   bitlinear_pack_weights_noalloc uses in place of a workspace.
 * - `stream` is a hipStream_t passed as void*; NULL selects the null stream.
 *   Every call only enqueues work on `stream`: it never synchronises the host.
 * - Arguments are validated on the host before any HIP call.  A failed check
 *   returns its bl_status code and records a message that
 *   bitlinear_last_error() returns (per thread).  A failed launch returns
 *   BL_ERR_HIP.  Faults inside a kernel surface at the caller's next
 *   synchronisation.  No C++ exception crosses this interface.
 * - Inputs must be finite; this is not checked on the device.
 * - Calls are thread-safe; calls on different streams may run concurrently.
 *
 * Numerical contract (the plain reading of the pages, fixed here):
 * - eps = 1e-5f is added to gamma before the weight division (eq. (1)) and
 *   floors a token's absmax before the activation division; Qb = 127.
 * - Every round-to-integer rounds half to even; the weight division, the
 *   activation scale 127/m and the product x * (127/m) are single IEEE
 *   binary32 operations.
 * - gamma is the exact sum of |W| rounded once to binary64, divided by N*K in
 *   binary64 and rounded to binary32, so it does not depend on any order.
 * - y = acc * gamma * max(absmax, eps) / 127, computed in binary32 (within
 *   1e-5 relative of the binary64 value; y is +0 exactly where acc is 0).
 *   Where a later binary32 step depends on y's bits (the gated ReLU^2 below),
 *   y is instead the binary64 value ((acc * gamma) * m) / 127, one rounding
 *   per operation, rounded to binary32.
 *
 * Packed weight layout (the pages fix only "four weights per byte"):
 *   code c = t + 1 in {0, 1, 2} (3 never occurs).  Row n of the N x K matrix
 *   occupies K/4 bytes at byte offset n*K/4.  The 16 weights
 *   k = 16g + 4j + i (j, i in 0..3) of group g form one little-endian 32-bit
 *   word at row byte offset 4g, weight k in bits [8i + 2j, 8i + 2j + 2).
 *   Hence (word >> 2j) & 0x03030303 holds the codes of k = 16g+4j .. 16g+4j+3
 *   in its four bytes, in order.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BITLINEAR_ABI_VERSION 3   /* 3: bitlinear_calib_read takes a layout */

/* Largest K accepted: keeps every |acc| <= 127*K below 2^24, so the int32
 * sum converts to binary32 exactly. */
#define BITLINEAR_MAX_K 131072

typedef enum {
  BL_OK = 0,
  BL_ERR_NULL = 1,      /* a required pointer is NULL */
  BL_ERR_SHAPE = 2,     /* T, N or K out of range, or K % 16 != 0 */
  BL_ERR_ALIGN = 3,     /* a pointer lacks the alignment stated below */
  BL_ERR_DTYPE = 4,     /* unknown activation dtype */
  BL_ERR_WORKSPACE = 5, /* workspace smaller than bitlinear_pack_workspace_bytes */
  BL_ERR_HIP = 6,       /* a HIP launch failed; the message names the error */
  BL_ERR_ARG = 7        /* another invalid argument (e.g. unknown algorithm) */
} bl_status;

typedef enum { BL_F32 = 0, BL_BF16 = 1 } bl_dtype;

typedef enum {
  BL_ALGO_AUTO = 0, /* decode kernel for T up to a limit set by the matrix's packed size
                       (64 up to 2 MB, 32 up to 16 MB, 6 beyond: measured crossovers),
                       else GEMM */
  BL_ALGO_GEMV = 1, /* streaming decode kernel, any T (tokens taken 64 at a time) */
  BL_ALGO_GEMM = 2, /* LDS-tiled int8 MFMA kernel, any T */
  BL_ALGO_LUT = 3   /* table-lookup decode kernel in the style of bitnet.cpp's TL1/TL2
                       ("微软 BitNet ...", section 1.3), any T (weights re-read per
                       token): a comparison design with the same results */,
  BL_ALGO_DOT4 = 4  /* decode kernel on packed int8 dot instructions (v_dot4) instead of
                       the matrix cores, any T (weights re-read per token): a comparison
                       design with the same results */
} bl_algo;

/* Version of this interface (BITLINEAR_ABI_VERSION). */
int bitlinear_abi_version(void);

/* Text of the last non-OK status returned on the calling thread ("" if none).
 * The pointer stays valid until the next call on the same thread. */
const char* bitlinear_last_error(void);

/* Largest T that BL_ALGO_AUTO sends to the decode (GEMV) kernel for any
 * matrix (64); larger matrices switch to the tiled kernel earlier (see
 * BL_ALGO_AUTO). */
int64_t bitlinear_gemv_max_tokens(void);

/* Bytes of device workspace that bitlinear_pack_weights needs for an N x K
 * matrix (a small constant: the exact-sum buckets of gamma). */
size_t bitlinear_pack_workspace_bytes(int64_t N, int64_t K);

/* Step A0: absmean ternarisation and 2-bit packing of one weight matrix.
 * Follows "BitNet解读", weight quantisation function: gamma = mean |W| over
 * all N*K entries (eq. (3)), t = RoundClip(W / (gamma + eps), -1, 1)
 * (eq. (1), (2)); packing follows the 2B4T report, section 5.1 (four ternary
 * values per 8-bit integer), in the layout stated at the top of this file.
 *
 *   w         [N, K] float32 latent weights, row-major, 16-byte aligned.
 *   N, K      1 <= N <= 2^26, 16 <= K <= BITLINEAR_MAX_K, K % 16 == 0.
 *   packed    [N, K/4] uint8 output, 16-byte aligned.
 *   gamma     [1] float32 output (device), 4-byte aligned.
 *   workspace device scratch of at least bitlinear_pack_workspace_bytes(N, K)
 *             bytes, 8-byte aligned; its contents are overwritten.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_WORKSPACE, BL_ERR_HIP. */
bl_status bitlinear_pack_weights(const float* w, int64_t N, int64_t K, uint8_t* packed,
                                 float* gamma, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* bitlinear_pack_weights without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The same kernels and results as
 * bitlinear_pack_weights; the gamma buckets live in a fixed 2 KiB array in the
 * library's device memory (256 x uint64, one copy per device, kept until the
 * process ends).  The call allocates nothing.  Every call on one device shares
 * that array and clears it first, so calls that overlap on one device (on
 * different streams, or from different threads without ordering) race and
 * may return a wrong gamma; calls on one stream are ordered and safe.
 *
 *   w, N, K, packed, gamma   as bitlinear_pack_weights; N*K <= 2^38, the most
 *            that the fixed buckets sum exactly (larger matrices: BL_ERR_SHAPE).
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_HIP (also when the
 * array's device address cannot be looked up). */
bl_status bitlinear_pack_weights_noalloc(const float* w, int64_t N, int64_t K, uint8_t* packed,
                                         float* gamma, void* stream);

/* Step A1: per-token absmax quantisation of activations to int8.
 * Follows "BitNet解读", activation quantisation (each token scaled into
 * [-Qb, Qb], no zero point) and the 2B4T report, section 2 (8-bit, absmax per
 * token).  Per row t: a = max_k |x[t,k]|, s = 127 / max(a, eps),
 * xq = clamp(round_half_even(x * s), -127, 127).
 *
 *   x        [T, K] activations of dtype x_dtype (BL_F32 or BL_BF16),
 *            row-major, 16-byte aligned.
 *   T, K     1 <= T <= 2^24, 16 <= K <= BITLINEAR_MAX_K, K % 16 == 0.
 *   xq       [T, K] int8 output, 16-byte aligned.
 *   absmax   [T] float32 output: a itself (not floored), 4-byte aligned.
 *   rowsum   [T] int32 output sum_k xq[t,k], or NULL to skip it.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_DTYPE, BL_ERR_HIP. */
bl_status bitlinear_quant_act(const void* x, int x_dtype, int64_t T, int64_t K, int8_t* xq,
                              float* absmax, int32_t* rowsum, void* stream);

/* The sub-layer norm in front of step A1, fused with it.  The 2B4T report
 * (section 2) puts subln before the quantised projections and drops every
 * bias; the explainer's component table lists it in place of RMSNorm /
 * LayerNorm.  No page gives its formula; it is taken here as an RMS norm with
 * a per-feature gain g and no bias, applied first, its output then quantised
 * by step A1.  Per token, in this order and precision:
 *   S        = sum_k x[t,k]^2, exact, rounded once to binary64 (no order of
 *              summation matters),
 *   ms       = RN32(RN64(S / K)),
 *   r        = RN32(1 / RN32(sqrt(RN32(ms + eps_n)))),
 *   x_hat    = RN32(RN32(x * g) * r),
 *   scale[t] = max_k |x_hat[t,k]|  (exact),
 *   xq[t,k]  = clamp(round_half_even(x_hat * RN32(127 / max(scale, eps))), -127, 127).
 * scale takes the place of absmax in bitlinear_forward.  Rows whose mean
 * square exceeds the binary32 range are outside the domain.
 *
 *   x        [T, K] activations of dtype x_dtype (BL_F32 or BL_BF16), 16-byte aligned.
 *   gain     [K] float32 per-feature gain (device), 16-byte aligned.
 *   eps_n    the norm's epsilon, finite and > 0 (1e-5 is this library's reading).
 *   T, K     1 <= T <= 2^24, 16 <= K <= BITLINEAR_MAX_K, K % 16 == 0.
 *   xq       [T, K] int8 output, 16-byte aligned.
 *   scale    [T] float32 output, 4-byte aligned.
 *   rowsum   [T] int32 output sum_k xq[t,k], or NULL.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_DTYPE, BL_ERR_ARG
 * (eps_n), BL_ERR_HIP. */
bl_status bitlinear_subln_quant_act(const void* x, int x_dtype, const float* gain, float eps_n,
                                    int64_t T, int64_t K, int8_t* xq, float* scale, int32_t* rowsum,
                                    void* stream);

/* Steps A2 and A3: y[t, n] = (sum_k t[n,k] * xq[t,k]) * gamma * max(absmax[t], eps) / 127.
 * The contraction follows "BitNet解读", computational efficiency (ternary
 * weights turn products into add, subtract or skip) and is exact in int32;
 * the rescale follows the bitnet.cpp post, section 1.1 (the scale factor).
 * Dispatches on T, N and K (BL_ALGO_AUTO); see bitlinear_forward_algo.
 *
 * The matrix-core kernels contract the stored codes c = t + 1 and remove
 * sum_k xq[t,k] from each token's sums afterwards.  With `rowsum` given they
 * take that sum from it, once per token; with NULL every kernel derives it
 * from the activations it reads.
 *
 *   packed   [N, K/4] uint8 from bitlinear_pack_weights, 16-byte aligned.
 *   gamma    [1] float32 (device) from bitlinear_pack_weights.
 *   xq       [T, K] int8 from bitlinear_quant_act, 16-byte aligned.
 *   absmax   [T] float32 from bitlinear_quant_act.
 *   rowsum   [T] int32 sum_k xq[t,k] as bitlinear_quant_act writes it, 4-byte
 *            aligned, or NULL.  Any other value gives wrong results (it is
 *            not checked).
 *   T, N, K  1 <= T <= 2^24, 1 <= N <= 2^26, 16 <= K <= BITLINEAR_MAX_K, K % 16 == 0.
 *   y        [T, N] float32 output, 4-byte aligned.
 *   acc      [T, N] int32 output of the exact sums, or NULL to skip it.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_HIP. */
bl_status bitlinear_forward(const uint8_t* packed, const float* gamma, const int8_t* xq,
                            const float* absmax, const int32_t* rowsum, int64_t T, int64_t N,
                            int64_t K, float* y, int32_t* acc, void* stream);

/* bitlinear_forward with an explicit kernel choice (a bl_algo value); the
 * results are identical for every choice (the table-lookup and packed-dot
 * kernels work on signed weights and do not read rowsum).  Errors as
 * bitlinear_forward, plus BL_ERR_ARG for an unknown algo. */
bl_status bitlinear_forward_algo(const uint8_t* packed, const float* gamma, const int8_t* xq,
                                 const float* absmax, const int32_t* rowsum, int64_t T, int64_t N,
                                 int64_t K, float* y, int32_t* acc, int algo, void* stream);

/* One problem of bitlinear_linear_grouped: a whole BitLinear forward. */
typedef struct bl_linear {
  const void* x;          /* [T, K] activations, dtype of the call, 16-byte aligned */
  const uint8_t* packed;  /* [N, K/4] from bitlinear_pack_weights, 16-byte aligned */
  const float* gamma;     /* [1] from bitlinear_pack_weights */
  int64_t N, K;           /* 1 <= N <= 2^26, 16 <= K <= BITLINEAR_MAX_K, K % 16 == 0 */
  float* y;               /* [T, N] output, 4-byte aligned */
  int8_t* xq;             /* [T, K] int8 activations (written), 16-byte aligned */
  float* absmax;          /* [T] token absmax (written) */
  int32_t* acc;           /* [T, N] exact int32 sums, or NULL */
} bl_linear;

/* Steps A1-A3 for `count` (1..8) independent BitLinear problems that share T
 * and the activation dtype: the same results as bitlinear_quant_act followed
 * by bitlinear_forward on each problem (same operations, same rounding), for
 * callers that run several projections of one layer back to back (e.g. the
 * query/key/value or gate/up projections of a decoder layer).  For decode
 * shapes (T <= 4, K % 64 == 0, T times K rounded up to a multiple of 256 at
 * most 32768, raw activation rows of at most 32 KiB when T > 1, and a modest
 * total of weight rows times K) one kernel
 * does all of it: each block quantises the activations it needs (one token:
 * from registers; more: from rows staged in LDS), then streams its weight
 * rows; otherwise the steps run per problem (act-quant, then the kernel that
 * bitlinear_forward would choose).
 *
 *   problems  HOST array of `count` descriptors (read during the call only).
 *   T         1 <= T <= 2^24 tokens, the same for every problem.
 *   x_dtype   BL_F32 or BL_BF16.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_DTYPE, BL_ERR_ARG
 * (count out of range), BL_ERR_HIP. */
bl_status bitlinear_linear_grouped(const bl_linear* problems, int count, int64_t T, int x_dtype,
                                   void* stream);

/* Step A0 for binary weights (+1 / -1, one bit each).  The original BitNet
 * has only these two values (the 2B4T explainer, section 2; "BitNet解读", on
 * the zero weight); no page gives the rule, which is read as the absmean
 * scheme with two levels: gamma = mean |W| over all N*K entries (eq. (3), as
 * bitlinear_pack_weights computes it), t = +1 where W >= 0 (either zero) and
 * -1 where W < 0.  Layout: row n at byte n*K/8; weight k = 32g + 4j + i of a
 * row is bit 8i + j of its little-endian 32-bit word g (bit 1 = +1).
 *
 *   w         [N, K] float32 latent weights, row-major, 16-byte aligned.
 *   N, K      1 <= N <= 2^26, 256 <= K <= 32768, K % 256 == 0.
 *   packed    [N, K/8] uint8 output, 16-byte aligned.
 *   gamma     [1] float32 output (device), 4-byte aligned.
 *   workspace device scratch of at least bitlinear_pack_workspace_bytes(N, K) bytes.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_WORKSPACE, BL_ERR_HIP. */
bl_status bitlinear_pack_weights_binary(const float* w, int64_t N, int64_t K, uint8_t* packed,
                                        float* gamma, void* workspace, size_t workspace_bytes,
                                        void* stream);

/* Steps A2 and A3 on binary weights: y[t, n] = (sum_k t[n,k] * xq[t,k]) *
 * gamma * max(absmax[t], eps) / 127 with t in {-1, +1}, exact in int32, as
 * bitlinear_forward.  BL_ALGO_AUTO takes the decode kernel for T <= 16 with
 * T*K <= 32768, else the tiled MFMA kernel; BL_ALGO_GEMV (the decode kernel,
 * tokens taken as many as fit at a time) and BL_ALGO_GEMM force one; results
 * are identical for every choice.
 *
 *   packed   [N, K/8] from bitlinear_pack_weights_binary, 16-byte aligned.
 *   gamma    [1] float32 (device).
 *   xq, absmax, y, acc   as bitlinear_forward.
 *   T, N, K  1 <= T <= 2^24, 1 <= N <= 2^26, 256 <= K <= 32768, K % 256 == 0,
 *            T*K < 2^31, N*K/32 < 2^31.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_ARG (BL_ALGO_LUT,
 * BL_ALGO_DOT4 or unknown), BL_ERR_HIP. */
bl_status bitlinear_forward_binary(const uint8_t* packed, const float* gamma, const int8_t* xq,
                                   const float* absmax, int64_t T, int64_t N, int64_t K, float* y,
                                   int32_t* acc, int algo, void* stream);

/* Row interleave of two packed matrices of the same shape, for
 * bitlinear_gated_relu2: out row 2i is row i of a, out row 2i + 1 row i of b
 * (four ternary weights per byte in each row, as bitlinear_pack_weights
 * writes them).  Each matrix keeps its own gamma.
 *
 *   a, b     [N, K/4] uint8 packed matrices (device), 4-byte aligned.
 *   N, K     1 <= N <= 2^25, 16 <= K <= BITLINEAR_MAX_K, K % 16 == 0.
 *   out      [2N, K/4] uint8 output (device), 4-byte aligned; must not overlap a or b.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_HIP. */
bl_status bitlinear_interleave_rows(const uint8_t* a, const uint8_t* b, int64_t N, int64_t K,
                                    uint8_t* out, void* stream);

/* The gate and up projections of one input (steps A1-A3 each) and the
 * squared-ReLU activation that the 2B4T report (section 2) puts in the
 * feed-forward sublayer, read as a gated unit and written as bfloat16 for the
 * down projection:
 *   g, u = step A3 of the gate and up sums in binary64, ((acc * gamma) * m)
 *       / 127 with m = max(absmax, eps), one rounding per operation, rounded
 *       to binary32,
 *   h[t,n] = bf16_round_nearest_even((max(g, 0) * max(g, 0)) * u)
 *       (two binary32 products in that order).
 * The activations are quantised once (step A1) and shared by both
 * projections; for decode shapes (T <= 4, K % 64 == 0, T times K rounded up
 * to a multiple of 256 at most 32768, raw rows of at most 32 KiB when T > 1,
 * and a modest total of weight rows times K) one kernel does everything, otherwise act-quant runs first and the
 * contraction kernel (chosen by T) writes h in its epilogue.  The gate/up
 * outputs are never stored in binary32.
 *
 *   x           [T, K] activations of dtype x_dtype (BL_F32 or BL_BF16), 16-byte aligned.
 *   packed_gu   [2N, K/4] from bitlinear_interleave_rows(gate, up), 16-byte aligned.
 *   gamma_gate, gamma_up   [1] float32 each (device), from bitlinear_pack_weights.
 *   T, N, K     1 <= T <= 2^24, 1 <= N <= 2^25 (outputs per token), 16 <= K <= BITLINEAR_MAX_K,
 *               K % 16 == 0.
 *   h           [T, N] bfloat16 output (uint16 bit patterns), 2-byte aligned.
 *   xq          [T, K] int8 activations (written), 16-byte aligned.
 *   absmax      [T] token absmax (written), 4-byte aligned.
 *   acc         [T, 2N] exact int32 sums, interleaved as the rows (gate, up), or NULL.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE, BL_ERR_ALIGN, BL_ERR_DTYPE, BL_ERR_HIP. */
bl_status bitlinear_gated_relu2(const void* x, int x_dtype, const uint8_t* packed_gu,
                                const float* gamma_gate, const float* gamma_up, int64_t T, int64_t N,
                                int64_t K, uint16_t* h, int8_t* xq, float* absmax, int32_t* acc,
                                void* stream);

/* ------------------------------------------------------------------------
 * Measurement helpers.  Not part of the forward: they measure, on the device
 * at hand, the ceilings that the forward's kernels are compared with (the
 * launch floor, the HBM read stream, the int8 matrix-core rate).  Errors as
 * for every call above; they touch no memory but their own arguments.
 * ------------------------------------------------------------------------ */

/* Entries (uint32 or int32) that the sink of the two calls below must hold. */
int64_t bitlinear_calib_sink_len(void);

/* One empty kernel on `stream`: the cost of a launch with no work. */
bl_status bitlinear_calib_empty(void* stream);

/* Layouts of bitlinear_calib_read: which 16-byte vectors a lane keeps in
 * flight (eight at a time). */
typedef enum {
  BL_READ_CHUNKS = 0, /* blocks take contiguous 32 KiB chunks; a lane's loads 4 KiB apart */
  BL_READ_STRIDE = 1  /* grid-stride loop; a lane's loads one grid (4 MiB) apart */
} bl_read_layout;

/* Reads the `bytes` bytes at `buf` (device, 16-byte aligned; `bytes` a
 * positive multiple of 16, at most 2^40) once, with 16-byte loads over a
 * grid of 1024 blocks of four waves that fills the device, in the given
 * bl_read_layout.  sink[w] for w < 4096 receives the XOR of the 32-bit words
 * that wave w read, so the XOR of those 4096 entries is the XOR of the whole
 * buffer.
 * Errors: BL_ERR_NULL, BL_ERR_SHAPE (bytes), BL_ERR_ARG (layout),
 * BL_ERR_ALIGN. */
bl_status bitlinear_calib_read(const void* buf, int64_t bytes, int layout, uint32_t* sink,
                               void* stream);

/* 4096 waves (four per SIMD on 256 CUs) each issue `iters` rounds of four
 * independent v_mfma_i32_32x32x32_i8 with every element of A and B equal to
 * the int8 value `byte`: 4 * iters * 4096 * 32768 int8 multiply-adds in
 * all (count two operations each for a TOP/s figure).  sink[w] for w < 4096
 * receives 4 * iters * 32 * byte^2 modulo 2^32 (as int32).
 * Errors: BL_ERR_NULL, BL_ERR_ARG (iters outside [1, 2^20], byte outside
 * [-128, 127]). */
bl_status bitlinear_calib_mfma(int64_t iters, int byte, int32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
