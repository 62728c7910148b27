// C ABI of libw4: argument validation, kernel selection, error reporting.
// Every check happens before any HIP call, so an invalid request enqueues
// nothing.  No exception leaves this file.
#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "w4_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_last_error[0] = '\0';
  return W4_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(W4_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxK = (int64_t)1 << 23;      // columns
constexpr int64_t kMaxElems = (int64_t)1 << 36;  // n*k, m*k, m*n
constexpr int64_t kMaxActTokens = (int64_t)1 << 24;  // quantize_act_int8: m < 2^24

// Shared checks of the weight-side arguments (shape, group, scale dtype).
int check_weights(const char* fn, int64_t n, int64_t k, int32_t g, int sz_dtype) {
  if (n < 0) return fail(W4_EINVAL, "%s: n = %lld < 0", fn, (long long)n);
  if (k <= 0) return fail(W4_EINVAL, "%s: k = %lld must be > 0", fn, (long long)k);
  if (g <= 0 || g % 32 != 0)
    return fail(W4_EINVAL, "%s: group_size = %d must be a positive multiple of 32", fn, g);
  if (k % g != 0)
    return fail(W4_EINVAL, "%s: k = %lld is not a multiple of group_size = %d", fn, (long long)k, g);
  if (sz_dtype != W4_F32 && sz_dtype != W4_F16)
    return fail(W4_EINVAL, "%s: scale dtype %d must be W4_F32 or W4_F16", fn, sz_dtype);
  // Size limits that keep every kernel's 32-bit tile offsets (up to 256 rows
  // of K elements) and launch sizes (under 2^32 work-items) in range for the
  // weight-side launches; quantize_act_int8 bounds its token count itself.
  if (k > kMaxK)
    return fail(W4_EINVAL, "%s: k = %lld is too large (at most %lld)", fn, (long long)k,
                (long long)kMaxK);
  if (n > kMaxElems / k)
    return fail(W4_EINVAL, "%s: n * k = %lld * %lld is too large", fn, (long long)n, (long long)k);
  return W4_OK;
}

// Shared checks of the token count against K and N (matmuls).
int check_tokens(const char* fn, int64_t m, int64_t k, int64_t n) {
  if (m < 0) return fail(W4_EINVAL, "%s: m = %lld < 0", fn, (long long)m);
  if (m > 0x7fffffffLL) return fail(W4_EINVAL, "%s: m = %lld is too large", fn, (long long)m);
  if (m > kMaxElems / k) return fail(W4_EINVAL, "%s: m * k is too large", fn);
  if (n > 0 && m > kMaxElems / n) return fail(W4_EINVAL, "%s: m * n is too large", fn);
  return W4_OK;
}

int check_ptr(const char* fn, const char* name, const void* p) {
  if (p == nullptr) return fail(W4_EINVAL, "%s: %s is NULL", fn, name);
  if (!aligned16(p)) return fail(W4_EINVAL, "%s: %s is not 16-byte aligned", fn, name);
  return W4_OK;
}

#define W4_TRY(expr)              \
  do {                            \
    const int rc_ = (expr);       \
    if (rc_ != W4_OK) return rc_; \
  } while (0)

}  // namespace

extern "C" {

const char* w4_status_string(int status) {
  switch (status) {
    case W4_OK: return "W4_OK: success";
    case W4_EINVAL: return "W4_EINVAL: invalid argument";
    case W4_EUNSUPPORTED: return "W4_EUNSUPPORTED: request not supported by this build";
    case W4_EHIP: return "W4_EHIP: HIP runtime error";
    default: return "unknown w4 status";
  }
}

const char* w4_last_error(void) { return g_last_error; }

const char* w4_version(void) { return "w4 0.1.0 gfx950"; }

static int quantize_pack_common(const char* fn, bool symmetric, const void* w, int w_dtype,
                                int64_t n, int64_t k, int32_t group_size, uint8_t* packed,
                                void* scales, void* zeros, int sz_dtype, hipStream_t stream) {
  W4_TRY(check_weights(fn, n, k, group_size, sz_dtype));
  if (w_dtype != W4_F32 && w_dtype != W4_BF16)
    return fail(W4_EINVAL, "%s: w dtype %d must be W4_F32 or W4_BF16", fn, w_dtype);
  if (n == 0) return ok();
  W4_TRY(check_ptr(fn, "w", w));
  W4_TRY(check_ptr(fn, "packed", packed));
  W4_TRY(check_ptr(fn, "scales", scales));
  W4_TRY(check_ptr(fn, "zeros", zeros));
  return hip_status(w4::launch_quantize_pack(w, w_dtype, n, k, group_size, packed, scales, zeros,
                                             sz_dtype, symmetric, stream),
                    fn);
}

int quantize_pack_int4(const void* w, int w_dtype, int64_t n, int64_t k, int32_t group_size,
                       uint8_t* packed, void* scales, void* zeros, int sz_dtype,
                       hipStream_t stream) {
  return quantize_pack_common("quantize_pack_int4", false, w, w_dtype, n, k, group_size, packed,
                              scales, zeros, sz_dtype, stream);
}

int quantize_pack_int4_sym(const void* w, int w_dtype, int64_t n, int64_t k, int32_t group_size,
                           uint8_t* packed, void* scales, void* zeros, int sz_dtype,
                           hipStream_t stream) {
  return quantize_pack_common("quantize_pack_int4_sym", true, w, w_dtype, n, k, group_size, packed,
                              scales, zeros, sz_dtype, stream);
}

static int quantize_pack_cal(const char* fn, int mode, double param, const void* w, int w_dtype,
                             int64_t n, int64_t k, int32_t group_size, uint8_t* packed, void* scales,
                             void* zeros, int sz_dtype, hipStream_t stream) {
  W4_TRY(check_weights(fn, n, k, group_size, sz_dtype));
  if (!w4::quantize_cal_fits(group_size))
    return fail(W4_EINVAL, "%s: group_size = %d is above the calibrators' limit of 1024", fn,
                (int)group_size);
  if (w_dtype != W4_F32 && w_dtype != W4_BF16)
    return fail(W4_EINVAL, "%s: w dtype %d must be W4_F32 or W4_BF16", fn, w_dtype);
  if (n == 0) return ok();
  W4_TRY(check_ptr(fn, "w", w));
  W4_TRY(check_ptr(fn, "packed", packed));
  W4_TRY(check_ptr(fn, "scales", scales));
  W4_TRY(check_ptr(fn, "zeros", zeros));
  return hip_status(w4::launch_quantize_pack_cal(w, w_dtype, n, k, group_size, mode, param, packed,
                                                 scales, zeros, sz_dtype, stream),
                    fn);
}

int quantize_pack_int4_sym_percentile(const void* w, int w_dtype, int64_t n, int64_t k,
                                      int32_t group_size, double percentile, uint8_t* packed,
                                      void* scales, void* zeros, int sz_dtype, hipStream_t stream) {
  static const char* fn = "quantize_pack_int4_sym_percentile";
  if (!(percentile > 0.0 && percentile <= 100.0))
    return fail(W4_EINVAL, "%s: percentile %g must lie in (0, 100]", fn, percentile);
  return quantize_pack_cal(fn, 0, percentile, w, w_dtype, n, k, group_size, packed, scales, zeros,
                           sz_dtype, stream);
}

int quantize_pack_int4_sym_mse(const void* w, int w_dtype, int64_t n, int64_t k, int32_t group_size,
                               int32_t candidates, uint8_t* packed, void* scales, void* zeros,
                               int sz_dtype, hipStream_t stream) {
  static const char* fn = "quantize_pack_int4_sym_mse";
  if (candidates < 2 || candidates > 65536)
    return fail(W4_EINVAL, "%s: candidates = %d must lie in [2, 65536]", fn, (int)candidates);
  return quantize_pack_cal(fn, 1, (double)candidates, w, w_dtype, n, k, group_size, packed, scales,
                           zeros, sz_dtype, stream);
}

static constexpr int64_t kGptqMaxK = 65536;

int gptq_hessian(const float* x, int64_t t, int64_t k, double* h, hipStream_t stream) {
  static const char* fn = "gptq_hessian";
  if (t < 1) return fail(W4_EINVAL, "%s: t = %lld calibration rows, at least 1 needed", fn, (long long)t);
  if (k < 1 || k > kGptqMaxK)
    return fail(W4_EINVAL, "%s: k = %lld must lie in [1, %lld]", fn, (long long)k, (long long)kGptqMaxK);
  if (t > kMaxElems / k) return fail(W4_EINVAL, "%s: t * k is too large", fn);
  W4_TRY(check_ptr(fn, "x", x));
  W4_TRY(check_ptr(fn, "h", h));
  return hip_status(w4::launch_gptq_hessian(x, t, (int)k, h, stream), fn);
}

int gptq_inverse_cholesky(double* h, int64_t k, double* u, int32_t* info, hipStream_t stream) {
  static const char* fn = "gptq_inverse_cholesky";
  if (k < 1 || k > kGptqMaxK)
    return fail(W4_EINVAL, "%s: k = %lld must lie in [1, %lld]", fn, (long long)k, (long long)kGptqMaxK);
  W4_TRY(check_ptr(fn, "h", h));
  W4_TRY(check_ptr(fn, "u", u));
  if (info == nullptr) return fail(W4_EINVAL, "%s: info is NULL", fn);
  if ((reinterpret_cast<uintptr_t>(info) & 3u) != 0) return fail(W4_EINVAL, "%s: info is not 4-byte aligned", fn);
  if ((const void*)h == (const void*)u) return fail(W4_EINVAL, "%s: h and u must be distinct", fn);
  return hip_status(w4::launch_gptq_inverse_cholesky(h, (int)k, u, info, stream), fn);
}

int gptq_quantize_pack_int4(float* w, const double* u, int64_t n, int64_t k, int32_t group_size,
                            int32_t symmetric, uint8_t* packed, void* scales, void* zeros,
                            int sz_dtype, hipStream_t stream) {
  static const char* fn = "gptq_quantize_pack_int4";
  W4_TRY(check_weights(fn, n, k, group_size, sz_dtype));
  if (!w4::gptq_group_ok(group_size))
    return fail(W4_EINVAL, "%s: group_size = %d must be 32, 64 or a multiple of 128", fn, (int)group_size);
  if (k > kGptqMaxK)
    return fail(W4_EINVAL, "%s: k = %lld must be at most %lld", fn, (long long)k, (long long)kGptqMaxK);
  if (n == 0) return ok();
  W4_TRY(check_ptr(fn, "w", w));
  W4_TRY(check_ptr(fn, "u", u));
  W4_TRY(check_ptr(fn, "packed", packed));
  W4_TRY(check_ptr(fn, "scales", scales));
  W4_TRY(check_ptr(fn, "zeros", zeros));
  return hip_status(w4::launch_gptq_quantize_pack(w, u, n, (int)k, group_size, symmetric != 0, packed,
                                                  scales, zeros, sz_dtype, stream),
                    fn);
}

int dequant_int4(const uint8_t* packed, const void* scales, const void* zeros, int sz_dtype,
                 int64_t n, int64_t k, int32_t group_size, void* w_out, int out_dtype,
                 hipStream_t stream) {
  static const char* fn = "dequant_int4";
  W4_TRY(check_weights(fn, n, k, group_size, sz_dtype));
  if (out_dtype != W4_F32 && out_dtype != W4_F16 && out_dtype != W4_BF16)
    return fail(W4_EINVAL, "%s: out dtype %d must be W4_F32, W4_F16 or W4_BF16", fn, out_dtype);
  if (n == 0) return ok();
  W4_TRY(check_ptr(fn, "packed", packed));
  W4_TRY(check_ptr(fn, "scales", scales));
  W4_TRY(check_ptr(fn, "zeros", zeros));
  W4_TRY(check_ptr(fn, "w_out", w_out));
  return hip_status(
      w4::launch_dequant(packed, scales, zeros, sz_dtype, n, k, group_size, w_out, out_dtype, stream),
      fn);
}

int quantize_act_int8(const void* x, int x_dtype, int64_t m, int64_t k, int8_t* xq,
                      float* x_scale, hipStream_t stream) {
  static const char* fn = "quantize_act_int8";
  if (x_dtype != W4_F32 && x_dtype != W4_BF16)
    return fail(W4_EINVAL, "%s: x dtype %d must be W4_F32 or W4_BF16", fn, x_dtype);
  if (k <= 0 || k % 8 != 0)
    return fail(W4_EINVAL, "%s: k = %lld must be a positive multiple of 8", fn, (long long)k);
  if (k > kMaxK)
    return fail(W4_EINVAL, "%s: k = %lld is too large (at most %lld)", fn, (long long)k,
                (long long)kMaxK);
  W4_TRY(check_tokens(fn, m, k, 0));
  // One workgroup of up to 1024 (m < 64) or 256 work-items per token: below
  // 2^24 tokens the launch stays under 2^32 work-items.
  if (m >= kMaxActTokens)
    return fail(W4_EINVAL, "%s: m = %lld is too large (at most %lld tokens)", fn, (long long)m,
                (long long)(kMaxActTokens - 1));
  if (m == 0) return ok();
  W4_TRY(check_ptr(fn, "x", x));
  W4_TRY(check_ptr(fn, "xq", xq));
  if (x_scale == nullptr) return fail(W4_EINVAL, "%s: x_scale is NULL", fn);
  if ((reinterpret_cast<uintptr_t>(x_scale) & 3u) != 0)
    return fail(W4_EINVAL, "%s: x_scale is not 4-byte aligned", fn);
  return hip_status(w4::launch_act_quant(x, x_dtype, m, k, xq, x_scale, stream), fn);
}

// Which kernel w4a16_matmul runs for a (validated) shape.
enum class W16Path { DOT2, QUAD, DECODE, GEMV, GEMM, GENERIC };


static W16Path w4a16_path(int x_dtype, int64_t m, int64_t k, int64_t n, int32_t group_size,
                          bool split_ok) {
  // Kernel choice (bf16 activations): one token, groups of at least 128, K up
  // to 12288 -> the dot2 GEMV; two to four tokens at K = 4096, groups of a
  // multiple of 32 -> the 4x4x4 matrix-core GEMV (Llama-7B [11008,4096] at
  // 2 / 3 / 4 tokens: 7.8 / 7.9 / 8.3 us against 8.3 / 8.9 / 9.3 us on the
  // LDS decode kernel); other K up to four tokens with the activations fitting
  // in LDS, groups of a multiple of 128 -> the LDS decode kernel; up to 128
  // tokens, groups of a multiple of 128 -> the MFMA GEMV (in launches of up
  // to 64 tokens), except that with a workspace, from 65 tokens on at K >=
  // 8192, shapes whose GEMM splits K take the split-K GEMM (the [4096, 11008]
  // down projection at 65 to 128 tokens: 37-39 us against 51-79 us); more
  // tokens -> the MFMA GEMM; everything else (fp32 activations, smaller
  // group sizes at few tokens) -> the general kernel.
  if (x_dtype == W4_BF16 && w4::dot2_fits(m, k, group_size)) return W16Path::DOT2;
  if (x_dtype == W4_BF16 && w4::quad_fits(m, k, group_size)) return W16Path::QUAD;
  if (x_dtype == W4_BF16 && m <= 4 && group_size % 128 == 0 && w4::decode_lds_fits(m, k))
    return W16Path::DECODE;
  const bool gemv = x_dtype == W4_BF16 && w4::gemv_mfma_fits(m, k, group_size);
  if (gemv && split_ok && m >= 65 && k >= 8192 && w4::gemm_workspace_bytes(m, k, n, group_size) > 0)
    return W16Path::GEMM;
  if (gemv) return W16Path::GEMV;
  if (x_dtype == W4_BF16 && w4::gemm_fits(m, k, group_size)) return W16Path::GEMM;
  return W16Path::GENERIC;
}

// ws / ws_bytes: the caller's workspace (w4a16_matmul_ws); use_scratch: the
// library's static scratch instead (w4a16_matmul_noalloc), looked up only
// after every argument has been validated.
static int w4a16_common(const char* fn, const void* x, int x_dtype, int64_t m, int64_t k,
                        const uint8_t* packed, const void* scales, const void* zeros, int sz_dtype,
                        int64_t n, int32_t group_size, void* y, int y_dtype, void* ws,
                        size_t ws_bytes, bool use_scratch, hipStream_t stream) {
  W4_TRY(check_weights(fn, n, k, group_size, sz_dtype));
  if (x_dtype != W4_F32 && x_dtype != W4_BF16)
    return fail(W4_EINVAL, "%s: x dtype %d must be W4_F32 or W4_BF16", fn, x_dtype);
  if (y_dtype != W4_F32 && y_dtype != W4_BF16)
    return fail(W4_EINVAL, "%s: y dtype %d must be W4_F32 or W4_BF16", fn, y_dtype);
  W4_TRY(check_tokens(fn, m, k, n));
  if (m == 0 || n == 0) return ok();
  W4_TRY(check_ptr(fn, "x", x));
  W4_TRY(check_ptr(fn, "packed", packed));
  W4_TRY(check_ptr(fn, "scales", scales));
  W4_TRY(check_ptr(fn, "zeros", zeros));
  W4_TRY(check_ptr(fn, "y", y));
  if (ws != nullptr && ws_bytes > 0 && !aligned16(ws))
    return fail(W4_EINVAL, "%s: workspace is not 16-byte aligned", fn);
  // the split-K GEMM is chosen only when its partials have room
  const size_t split_bytes = (x_dtype == W4_BF16) ? w4::gemm_workspace_bytes(m, k, n, group_size) : 0;
  const bool split_ok = split_bytes > 0 && (use_scratch || (ws != nullptr && ws_bytes >= split_bytes));
  const W16Path path = w4a16_path(x_dtype, m, k, n, group_size, split_ok);
  if (use_scratch && path == W16Path::GEMM) {
    // only a shape that splits K needs the scratch
    ws_bytes = w4::gemm_workspace_bytes(m, k, n, group_size);
    if (ws_bytes > w4::kSplitKMaxBytes)
      return fail(W4_EINVAL, "%s: this shape needs %zu bytes of scratch, above the library's %zu", fn,
                  ws_bytes, w4::kSplitKMaxBytes);
    if (ws_bytes > 0) {
      const hipError_t e = w4::scratch_address(&ws);
      if (e != hipSuccess) return hip_status(e, fn);
    }
  }
  switch (path) {
    case W16Path::DOT2:
      return hip_status(w4::launch_w4a16_dot2(x, m, k, packed, scales, zeros, sz_dtype, n,
                                              group_size, y, y_dtype, stream),
                        fn);
    case W16Path::QUAD:
      return hip_status(w4::launch_w4a16_quad(x, m, k, packed, scales, zeros, sz_dtype, n,
                                              group_size, y, y_dtype, stream),
                        fn);
    case W16Path::DECODE:
      return hip_status(w4::launch_w4a16_decode(x, m, k, packed, scales, zeros, sz_dtype, n,
                                                group_size, y, y_dtype, stream),
                        fn);
    case W16Path::GEMV:
      return hip_status(w4::launch_w4a16_gemv(x, m, k, packed, scales, zeros, sz_dtype, n,
                                              group_size, y, y_dtype, stream),
                        fn);
    case W16Path::GEMM:
      return hip_status(w4::launch_w4a16_gemm(x, m, k, packed, scales, zeros, sz_dtype, n,
                                              group_size, y, y_dtype, ws, ws_bytes, stream),
                        fn);
    default:
      return hip_status(w4::launch_w4a16_generic(x, x_dtype, m, k, packed, scales, zeros, sz_dtype,
                                                 n, group_size, y, y_dtype, stream),
                        fn);
  }
}

int w4a16_matmul(const void* x, int x_dtype, int64_t m, int64_t k, const uint8_t* packed,
                 const void* scales, const void* zeros, int sz_dtype, int64_t n,
                 int32_t group_size, void* y, int y_dtype, hipStream_t stream) {
  return w4a16_common("w4a16_matmul", x, x_dtype, m, k, packed, scales, zeros, sz_dtype, n,
                      group_size, y, y_dtype, nullptr, 0, false, stream);
}

int w4a16_matmul_noalloc(const void* x, int x_dtype, int64_t m, int64_t k, const uint8_t* packed,
                         const void* scales, const void* zeros, int sz_dtype, int64_t n,
                         int32_t group_size, void* y, int y_dtype, hipStream_t stream) {
  return w4a16_common("w4a16_matmul_noalloc", x, x_dtype, m, k, packed, scales, zeros, sz_dtype, n,
                      group_size, y, y_dtype, nullptr, 0, true, stream);
}

size_t w4a16_matmul_workspace_size(int64_t m, int64_t k, int64_t n, int32_t group_size,
                                   int x_dtype) {
  // Shapes the other entry points would reject need no workspace.
  if (m <= 0 || n <= 0 || k <= 0 || k > kMaxK || group_size <= 0 || group_size % 32 != 0 ||
      k % group_size != 0 || n > kMaxElems / k || m > 0x7fffffffLL || m > kMaxElems / k ||
      m > kMaxElems / n)
    return 0;
  if (w4a16_path(x_dtype, m, k, n, group_size, true) != W16Path::GEMM) return 0;
  return w4::gemm_workspace_bytes(m, k, n, group_size);
}

int w4a16_matmul_ws(const void* x, int x_dtype, int64_t m, int64_t k, const uint8_t* packed,
                    const void* scales, const void* zeros, int sz_dtype, int64_t n,
                    int32_t group_size, void* y, int y_dtype, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  return w4a16_common("w4a16_matmul_ws", x, x_dtype, m, k, packed, scales, zeros, sz_dtype, n,
                      group_size, y, y_dtype, workspace, workspace_bytes, false, stream);
}

// ws / ws_bytes: the caller's workspace (w4a8_matmul_ws), or none.
static int w4a8_common(const char* fn, const int8_t* xq, const float* x_scale, int64_t m, int64_t k,
                       const uint8_t* packed, const void* scales, const void* zeros, int sz_dtype,
                       int64_t n, int32_t group_size, void* y, int y_dtype, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  W4_TRY(check_weights(fn, n, k, group_size, sz_dtype));
  if (y_dtype != W4_F32 && y_dtype != W4_BF16)
    return fail(W4_EINVAL, "%s: y dtype %d must be W4_F32 or W4_BF16", fn, y_dtype);
  W4_TRY(check_tokens(fn, m, k, n));
  if (m == 0 || n == 0) return ok();
  W4_TRY(check_ptr(fn, "xq", xq));
  W4_TRY(check_ptr(fn, "packed", packed));
  W4_TRY(check_ptr(fn, "scales", scales));
  W4_TRY(check_ptr(fn, "zeros", zeros));
  W4_TRY(check_ptr(fn, "y", y));
  if (x_scale == nullptr) return fail(W4_EINVAL, "%s: x_scale is NULL", fn);
  if ((reinterpret_cast<uintptr_t>(x_scale) & 3u) != 0)
    return fail(W4_EINVAL, "%s: x_scale is not 4-byte aligned", fn);
  if (ws != nullptr && ws_bytes > 0 && !aligned16(ws))
    return fail(W4_EINVAL, "%s: workspace is not 16-byte aligned", fn);
  // Kernel choice: one to four tokens, group 128, K a multiple of 2048 up to
  // 8192 -> the dot4 GEMV; up to 16 tokens, groups of a multiple of 128 ->
  // the int8 MFMA GEMV; more tokens -> the int8 MFMA GEMM (split K over the
  // workspace when its tiles would leave most of the GPU idle); everything
  // else -> the general kernel.
  if (w4::w4a8_gemv_fits(m, k, group_size))
    return hip_status(w4::launch_w4a8_gemv(xq, x_scale, m, k, packed, scales, zeros, sz_dtype, n,
                                           group_size, y, y_dtype, stream),
                      fn);
  if (w4::w4a8_gemv_mfma_fits(m, k, group_size))
    return hip_status(w4::launch_w4a8_gemv_mfma(xq, x_scale, m, k, packed, scales, zeros, sz_dtype,
                                                n, group_size, y, y_dtype, stream),
                      fn);
  if (w4::w4a8_gemm_fits(m, k, group_size))
    return hip_status(w4::launch_w4a8_gemm(xq, x_scale, m, k, packed, scales, zeros, sz_dtype, n,
                                           group_size, y, y_dtype, ws, ws_bytes, stream),
                      fn);
  return hip_status(w4::launch_w4a8_generic(xq, x_scale, m, k, packed, scales, zeros, sz_dtype, n,
                                            group_size, y, y_dtype, stream),
                    fn);
}

int w4a8_matmul(const int8_t* xq, const float* x_scale, int64_t m, int64_t k,
                const uint8_t* packed, const void* scales, const void* zeros, int sz_dtype,
                int64_t n, int32_t group_size, void* y, int y_dtype, hipStream_t stream) {
  return w4a8_common("w4a8_matmul", xq, x_scale, m, k, packed, scales, zeros, sz_dtype, n, group_size,
                     y, y_dtype, nullptr, 0, stream);
}

size_t w4a8_matmul_workspace_size(int64_t m, int64_t k, int64_t n, int32_t group_size) {
  // Shapes the other entry points would reject need no workspace.
  if (m <= 0 || n <= 0 || k <= 0 || k > kMaxK || group_size <= 0 || group_size % 32 != 0 ||
      k % group_size != 0 || n > kMaxElems / k || m > 0x7fffffffLL || m > kMaxElems / k ||
      m > kMaxElems / n)
    return 0;
  if (w4::w4a8_gemv_fits(m, k, group_size) || w4::w4a8_gemv_mfma_fits(m, k, group_size)) return 0;
  return w4::w4a8_gemm_workspace_bytes(m, k, n, group_size);
}

int w4a8_matmul_ws(const int8_t* xq, const float* x_scale, int64_t m, int64_t k,
                   const uint8_t* packed, const void* scales, const void* zeros, int sz_dtype,
                   int64_t n, int32_t group_size, void* y, int y_dtype, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  return w4a8_common("w4a8_matmul_ws", xq, x_scale, m, k, packed, scales, zeros, sz_dtype, n,
                     group_size, y, y_dtype, workspace, workspace_bytes, stream);
}

}  // extern "C"
