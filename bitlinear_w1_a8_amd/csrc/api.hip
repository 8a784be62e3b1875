// C ABI of libbitlinear (declared in include/bitlinear.h): argument checks on
// the host, then kernel launches on the caller's stream.
#include <stdio.h>
#include <stdarg.h>
#include <string>

#include "bitlinear.h"
#include <cmath>

#include "bl_internal.h"

namespace {

thread_local std::string g_last_error;

constexpr int64_t kMaxT = int64_t(1) << 24;
constexpr int64_t kMaxN = int64_t(1) << 26;
constexpr int64_t kMaxNK = int64_t(1) << 38;  // keeps every gamma bucket below 2^62
constexpr int64_t kMaxTN = int64_t(1) << 36;  // y up to 256 GiB
constexpr int64_t kMaxBinaryK = 32768;         // int8 rows of the binary decode kernel fit LDS

bl_status fail(bl_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bl_status check_k(const char* fn, int64_t k) {
  if (k < 16 || k > BITLINEAR_MAX_K || k % 16 != 0)
    return fail(BL_ERR_SHAPE, "%s: K=%lld must be a multiple of 16 in [16, %d]", fn,
                (long long)k, BITLINEAR_MAX_K);
  return BL_OK;
}

bl_status launched(const char* fn, hipError_t e) {
  if (e != hipSuccess) return fail(BL_ERR_HIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
  g_last_error.clear();
  return BL_OK;
}

}  // namespace

extern "C" {

int bitlinear_abi_version(void) { return BITLINEAR_ABI_VERSION; }

const char* bitlinear_last_error(void) { return g_last_error.c_str(); }

int64_t bitlinear_gemv_max_tokens(void) { return bl::kGemvMaxTokens; }

size_t bitlinear_pack_workspace_bytes(int64_t N, int64_t K) {
  (void)N;
  (void)K;
  return bl::kPackWorkspaceBytes;
}

bl_status bitlinear_pack_weights(const float* w, int64_t N, int64_t K, uint8_t* packed, float* gamma,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "bitlinear_pack_weights";
  if (!w || !packed || !gamma || !workspace) return fail(BL_ERR_NULL, "%s: NULL pointer argument", fn);
  if (bl_status rc = check_k(fn, K)) return rc;
  if (N < 1 || N > kMaxN || N * K > kMaxNK)
    return fail(BL_ERR_SHAPE, "%s: N=%lld out of range", fn, (long long)N);
  if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(gamma, 4) || !aligned(workspace, 8))
    return fail(BL_ERR_ALIGN, "%s: w and packed need 16-byte, gamma 4-byte, workspace 8-byte alignment", fn);
  if (workspace_bytes < bl::kPackWorkspaceBytes)
    return fail(BL_ERR_WORKSPACE, "%s: workspace of %zu bytes, need %zu", fn, workspace_bytes,
                bl::kPackWorkspaceBytes);
  return launched(fn, bl::launch_pack(w, N, K, packed, gamma,
                                      static_cast<unsigned long long*>(workspace),
                                      static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_pack_weights_noalloc(const float* w, int64_t N, int64_t K, uint8_t* packed,
                                         float* gamma, void* stream) {
  const char* fn = "bitlinear_pack_weights_noalloc";
  if (!w || !packed || !gamma) return fail(BL_ERR_NULL, "%s: NULL pointer argument", fn);
  if (bl_status rc = check_k(fn, K)) return rc;
  if (N < 1 || N > kMaxN || N * K > kMaxNK)
    return fail(BL_ERR_SHAPE, "%s: N=%lld, K=%lld: N*K above 2^38 would overflow the %d "
                "fixed buckets", fn, (long long)N, (long long)K, bl::kGammaBuckets);
  if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(gamma, 4))
    return fail(BL_ERR_ALIGN, "%s: w and packed need 16-byte, gamma 4-byte alignment", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned long long* buckets = nullptr;
  const hipError_t e = bl::scratch_buckets(s, &buckets);
  if (e != hipSuccess)
    return fail(BL_ERR_HIP, "%s: device scratch lookup failed: %s", fn, hipGetErrorString(e));
  return launched(fn, bl::launch_pack(w, N, K, packed, gamma, buckets, s));
}

bl_status bitlinear_quant_act(const void* x, int x_dtype, int64_t T, int64_t K, int8_t* xq,
                              float* absmax, int32_t* rowsum, void* stream) {
  const char* fn = "bitlinear_quant_act";
  if (!x || !xq || !absmax) return fail(BL_ERR_NULL, "%s: NULL pointer argument", fn);
  if (x_dtype != BL_F32 && x_dtype != BL_BF16)
    return fail(BL_ERR_DTYPE, "%s: unknown x_dtype %d", fn, x_dtype);
  if (bl_status rc = check_k(fn, K)) return rc;
  if (T < 1 || T > kMaxT) return fail(BL_ERR_SHAPE, "%s: T=%lld out of range", fn, (long long)T);
  if (!aligned(x, 16) || !aligned(xq, 16) || !aligned(absmax, 4) || (rowsum && !aligned(rowsum, 4)))
    return fail(BL_ERR_ALIGN, "%s: x and xq need 16-byte, absmax and rowsum 4-byte alignment", fn);
  return launched(fn, bl::launch_quant(x, x_dtype == BL_BF16, T, K, xq, absmax, rowsum,
                                       static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_subln_quant_act(const void* x, int x_dtype, const float* gain, float eps_n,
                                    int64_t T, int64_t K, int8_t* xq, float* scale, int32_t* rowsum,
                                    void* stream) {
  const char* fn = "bitlinear_subln_quant_act";
  if (!x || !gain || !xq || !scale) return fail(BL_ERR_NULL, "%s: NULL pointer argument", fn);
  if (x_dtype != BL_F32 && x_dtype != BL_BF16)
    return fail(BL_ERR_DTYPE, "%s: unknown x_dtype %d", fn, x_dtype);
  if (!(eps_n > 0.0f) || !std::isfinite(eps_n))
    return fail(BL_ERR_ARG, "%s: eps_n must be finite and > 0", fn);
  if (bl_status rc = check_k(fn, K)) return rc;
  if (T < 1 || T > kMaxT) return fail(BL_ERR_SHAPE, "%s: T=%lld out of range", fn, (long long)T);
  if (!aligned(x, 16) || !aligned(gain, 16) || !aligned(xq, 16) || !aligned(scale, 4) ||
      (rowsum && !aligned(rowsum, 4)))
    return fail(BL_ERR_ALIGN, "%s: x, gain and xq need 16-byte, scale and rowsum 4-byte alignment",
                fn);
  return launched(fn, bl::launch_subln_quant(x, x_dtype == BL_BF16, gain, eps_n, T, K, xq, scale,
                                             rowsum, static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_forward_algo(const uint8_t* packed, const float* gamma, const int8_t* xq,
                                 const float* absmax, const int32_t* rowsum, int64_t T, int64_t N,
                                 int64_t K, float* y, int32_t* acc, int algo, void* stream) {
  const char* fn = "bitlinear_forward";
  if (!packed || !gamma || !xq || !absmax || !y)
    return fail(BL_ERR_NULL, "%s: NULL pointer argument", fn);
  if (bl_status rc = check_k(fn, K)) return rc;
  if (T < 1 || T > kMaxT) return fail(BL_ERR_SHAPE, "%s: T=%lld out of range", fn, (long long)T);
  if (N < 1 || N > kMaxN || T * N > kMaxTN)
    return fail(BL_ERR_SHAPE, "%s: N=%lld out of range", fn, (long long)N);
  if (!aligned(packed, 16) || !aligned(xq, 16) || !aligned(gamma, 4) || !aligned(absmax, 4) ||
      !aligned(y, 4) || (acc && !aligned(acc, 4)) || (rowsum && !aligned(rowsum, 4)))
    return fail(BL_ERR_ALIGN, "%s: packed and xq need 16-byte, the others 4-byte alignment", fn);
  if (algo == BL_ALGO_AUTO) algo = bl::auto_algo(T, N, K);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (algo == BL_ALGO_GEMV)
    return launched(fn, bl::launch_gemv(packed, gamma, xq, absmax, rowsum, T, N, K, y, acc, s));
  if (algo == BL_ALGO_GEMM)
    return launched(fn, bl::launch_gemm(packed, gamma, xq, absmax, rowsum, T, N, K, y, acc, s));
  if (algo == BL_ALGO_LUT)
    return launched(fn, bl::launch_gemv_lut(packed, gamma, xq, absmax, T, N, K, y, acc, s));
  if (algo == BL_ALGO_DOT4)
    return launched(fn, bl::launch_gemv_dot4(packed, gamma, xq, absmax, T, N, K, y, acc, s));
  return fail(BL_ERR_ARG, "%s: unknown algo %d", fn, algo);
}

bl_status bitlinear_linear_grouped(const bl_linear* problems, int count, int64_t T, int x_dtype,
                                   void* stream) {
  const char* fn = "bitlinear_linear_grouped";
  if (!problems) return fail(BL_ERR_NULL, "%s: NULL problems array", fn);
  if (count < 1 || count > 8) return fail(BL_ERR_ARG, "%s: count=%d must be in [1, 8]", fn, count);
  if (x_dtype != BL_F32 && x_dtype != BL_BF16)
    return fail(BL_ERR_DTYPE, "%s: unknown x_dtype %d", fn, x_dtype);
  if (T < 1 || T > kMaxT) return fail(BL_ERR_SHAPE, "%s: T=%lld out of range", fn, (long long)T);
  for (int i = 0; i < count; ++i) {
    const bl_linear& q = problems[i];
    if (!q.x || !q.packed || !q.gamma || !q.y || !q.xq || !q.absmax)
      return fail(BL_ERR_NULL, "%s: problem %d: NULL pointer argument", fn, i);
    if (bl_status rc = check_k(fn, q.K)) return rc;
    if (q.N < 1 || q.N > kMaxN || T * q.N > kMaxTN)
      return fail(BL_ERR_SHAPE, "%s: problem %d: N=%lld out of range", fn, i, (long long)q.N);
    if (!aligned(q.x, 16) || !aligned(q.packed, 16) || !aligned(q.xq, 16) ||
        !aligned(q.gamma, 4) || !aligned(q.y, 4) || !aligned(q.absmax, 4) ||
        (q.acc && !aligned(q.acc, 4)))
      return fail(BL_ERR_ALIGN, "%s: problem %d: x, packed and xq need 16-byte, the others "
                  "4-byte alignment", fn, i);
  }
  return launched(fn, bl::launch_linear_group(problems, count, T, x_dtype == BL_BF16,
                                              static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_pack_weights_binary(const float* w, int64_t N, int64_t K, uint8_t* packed,
                                        float* gamma, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  const char* fn = "bitlinear_pack_weights_binary";
  if (!w || !packed || !gamma || !workspace) return fail(BL_ERR_NULL, "%s: NULL pointer argument", fn);
  if (K < 256 || K > kMaxBinaryK || K % 256 != 0)
    return fail(BL_ERR_SHAPE, "%s: K=%lld must be a multiple of 256 in [256, %lld]", fn,
                (long long)K, (long long)kMaxBinaryK);
  if (N < 1 || N > kMaxN || N * K > kMaxNK)
    return fail(BL_ERR_SHAPE, "%s: N=%lld out of range", fn, (long long)N);
  if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(gamma, 4) || !aligned(workspace, 8))
    return fail(BL_ERR_ALIGN, "%s: w and packed need 16-byte, gamma 4-byte, workspace 8-byte alignment", fn);
  if (workspace_bytes < bl::kPackWorkspaceBytes)
    return fail(BL_ERR_WORKSPACE, "%s: workspace of %zu bytes, need %zu", fn, workspace_bytes,
                bl::kPackWorkspaceBytes);
  return launched(fn, bl::launch_pack_binary(w, N, K, packed, gamma,
                                             static_cast<unsigned long long*>(workspace),
                                             static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_forward_binary(const uint8_t* packed, const float* gamma, const int8_t* xq,
                                   const float* absmax, int64_t T, int64_t N, int64_t K, float* y,
                                   int32_t* acc, int algo, void* stream) {
  const char* fn = "bitlinear_forward_binary";
  if (!packed || !gamma || !xq || !absmax || !y)
    return fail(BL_ERR_NULL, "%s: NULL pointer argument", fn);
  if (K < 256 || K > kMaxBinaryK || K % 256 != 0)
    return fail(BL_ERR_SHAPE, "%s: K=%lld must be a multiple of 256 in [256, %lld]", fn,
                (long long)K, (long long)kMaxBinaryK);
  if (T < 1 || T > kMaxT) return fail(BL_ERR_SHAPE, "%s: T=%lld out of range", fn, (long long)T);
  if (N < 1 || N > kMaxN || T * N > kMaxTN || T * K >= (int64_t(1) << 31) ||
      N * (K / 32) >= (int64_t(1) << 31))
    return fail(BL_ERR_SHAPE, "%s: N=%lld out of range", fn, (long long)N);
  if (!aligned(packed, 16) || !aligned(xq, 16) || !aligned(gamma, 4) || !aligned(absmax, 4) ||
      !aligned(y, 4) || (acc && !aligned(acc, 4)))
    return fail(BL_ERR_ALIGN, "%s: packed and xq need 16-byte, the others 4-byte alignment", fn);
  if (algo != BL_ALGO_AUTO && algo != BL_ALGO_GEMV && algo != BL_ALGO_GEMM)
    return fail(BL_ERR_ARG, "%s: algo %d not available for binary weights", fn, algo);  // LUT, DOT4
  return launched(fn, bl::launch_forward_binary(packed, gamma, xq, absmax, T, N, K, y, acc, algo,
                                                static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_interleave_rows(const uint8_t* a, const uint8_t* b, int64_t N, int64_t K,
                                    uint8_t* out, void* stream) {
  const char* fn = "bitlinear_interleave_rows";
  if (!a || !b || !out) return fail(BL_ERR_NULL, "%s: NULL pointer argument", fn);
  if (bl_status rc = check_k(fn, K)) return rc;
  if (N < 1 || 2 * N > kMaxN || 2 * N * K > kMaxNK)
    return fail(BL_ERR_SHAPE, "%s: N=%lld out of range", fn, (long long)N);
  if (!aligned(a, 4) || !aligned(b, 4) || !aligned(out, 4))
    return fail(BL_ERR_ALIGN, "%s: a, b and out need 4-byte alignment", fn);
  return launched(fn, bl::launch_interleave(a, b, N, K, out, static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_gated_relu2(const void* x, int x_dtype, const uint8_t* packed_gu,
                                const float* gamma_gate, const float* gamma_up, int64_t T, int64_t N,
                                int64_t K, uint16_t* h, int8_t* xq, float* absmax, int32_t* acc,
                                void* stream) {
  const char* fn = "bitlinear_gated_relu2";
  if (!x || !packed_gu || !gamma_gate || !gamma_up || !h || !xq || !absmax)
    return fail(BL_ERR_NULL, "%s: NULL pointer argument", fn);
  if (x_dtype != BL_F32 && x_dtype != BL_BF16)
    return fail(BL_ERR_DTYPE, "%s: unknown x_dtype %d", fn, x_dtype);
  if (bl_status rc = check_k(fn, K)) return rc;
  if (T < 1 || T > kMaxT) return fail(BL_ERR_SHAPE, "%s: T=%lld out of range", fn, (long long)T);
  if (N < 1 || 2 * N > kMaxN || T * 2 * N > kMaxTN)
    return fail(BL_ERR_SHAPE, "%s: N=%lld out of range", fn, (long long)N);
  if (!aligned(x, 16) || !aligned(packed_gu, 16) || !aligned(xq, 16) || !aligned(gamma_gate, 4) ||
      !aligned(gamma_up, 4) || !aligned(absmax, 4) || !aligned(h, 2) || (acc && !aligned(acc, 4)))
    return fail(BL_ERR_ALIGN, "%s: x, packed_gu and xq need 16-byte, h 2-byte, the others "
                "4-byte alignment", fn);
  return launched(fn, bl::launch_gated(x, x_dtype == BL_BF16, packed_gu, gamma_gate, gamma_up, T,
                                       2 * N, K, h, xq, absmax, acc,
                                       static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_forward(const uint8_t* packed, const float* gamma, const int8_t* xq,
                            const float* absmax, const int32_t* rowsum, int64_t T, int64_t N,
                            int64_t K, float* y, int32_t* acc, void* stream) {
  return bitlinear_forward_algo(packed, gamma, xq, absmax, rowsum, T, N, K, y, acc, BL_ALGO_AUTO,
                                stream);
}

int64_t bitlinear_calib_sink_len(void) { return bl::kCalibSinkLen; }

bl_status bitlinear_calib_empty(void* stream) {
  return launched("bitlinear_calib_empty", bl::launch_calib_empty(static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_calib_read(const void* buf, int64_t bytes, int layout, uint32_t* sink,
                               void* stream) {
  const char* fn = "bitlinear_calib_read";
  if (!buf || !sink) return fail(BL_ERR_NULL, "%s: NULL pointer argument", fn);
  if (bytes < 16 || bytes % 16 != 0 || bytes > (int64_t(1) << 40))
    return fail(BL_ERR_SHAPE, "%s: bytes=%lld must be a positive multiple of 16, at most 2^40", fn,
                (long long)bytes);
  if (layout != BL_READ_CHUNKS && layout != BL_READ_STRIDE)
    return fail(BL_ERR_ARG, "%s: unknown layout %d (BL_READ_CHUNKS or BL_READ_STRIDE)", fn, layout);
  if (!aligned(buf, 16) || !aligned(sink, 4))
    return fail(BL_ERR_ALIGN, "%s: buf needs 16-byte, sink 4-byte alignment", fn);
  return launched(fn, bl::launch_calib_read(buf, bytes, layout, sink,
                                            static_cast<hipStream_t>(stream)));
}

bl_status bitlinear_calib_mfma(int64_t iters, int byte, int32_t* sink, void* stream) {
  const char* fn = "bitlinear_calib_mfma";
  if (!sink) return fail(BL_ERR_NULL, "%s: NULL pointer argument", fn);
  if (iters < 1 || iters > (int64_t(1) << 20) || byte < -128 || byte > 127)
    return fail(BL_ERR_ARG, "%s: iters=%lld must be in [1, 2^20] and byte=%d in [-128, 127]", fn,
                (long long)iters, byte);
  if (!aligned(sink, 4)) return fail(BL_ERR_ALIGN, "%s: sink needs 4-byte alignment", fn);
  return launched(fn, bl::launch_calib_mfma((int)iters, byte, sink,
                                            static_cast<hipStream_t>(stream)));
}

}  // extern "C"
