// Internal launcher interface between the C ABI (api.cpp) and the kernels.
// Launchers assume validated arguments and enqueue on the given stream.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include <atomic>

#include "../../include/w4.h"

namespace w4 {

// Runs set() (an idempotent per-device setting such as a kernel's dynamic-LDS
// limit) once for the current device and remembers success in `done`, one bit
// per device.  Concurrent first calls may both run set(); that is harmless.
// Devices past 63 are set on every call.
template <typename F>
hipError_t once_per_device(std::atomic<uint64_t>& done, F set) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (1ull << dev) : 0ull;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = set();
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

hipError_t launch_quantize_pack(const void* w, int w_dtype, int64_t n, int64_t k, int g,
                                uint8_t* packed, void* scales, void* zeros, int sz_dtype,
                                bool symmetric, hipStream_t st);
// Calibrated symmetric quantize + pack: mode 0 = percentile (param = p in
// (0, 100]), mode 1 = MSE search (param = candidates, >= 2); g <= 1024.
bool quantize_cal_fits(int g);
hipError_t launch_quantize_pack_cal(const void* w, int w_dtype, int64_t n, int64_t k, int g, int mode,
                                    double param, uint8_t* packed, void* scales, void* zeros,
                                    int sz_dtype, hipStream_t st);
// GPTQ ([P4] Step 3): Hessian, inverse Cholesky factor, column sweep.
bool gptq_group_ok(int g);
hipError_t launch_gptq_hessian(const float* x, int64_t t, int k, double* h, hipStream_t st);
hipError_t launch_gptq_inverse_cholesky(double* h, int k, double* u, int* info, hipStream_t st);
hipError_t launch_gptq_quantize_pack(float* w, const double* u, int64_t n, int k, int g, bool symmetric,
                                     uint8_t* packed, void* scales, void* zeros, int sz_dtype,
                                     hipStream_t st);
hipError_t launch_dequant(const uint8_t* packed, const void* scales, const void* zeros,
                          int sz_dtype, int64_t n, int64_t k, int g, void* out, int out_dtype,
                          hipStream_t st);
hipError_t launch_act_quant(const void* x, int x_dtype, int64_t m, int64_t k, int8_t* xq,
                            float* x_scale, hipStream_t st);
hipError_t launch_w4a16_generic(const void* x, int x_dtype, int64_t m, int64_t k,
                                const uint8_t* packed, const void* scales, const void* zeros,
                                int sz_dtype, int64_t n, int g, void* y, int y_dtype,
                                hipStream_t st);
hipError_t launch_w4a16_decode(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                               const void* scales, const void* zeros, int sz_dtype, int64_t n,
                               int g, void* y, int y_dtype, hipStream_t st);
bool decode_lds_fits(int64_t m, int64_t k);
hipError_t launch_w4a16_dot2(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                             const void* scales, const void* zeros, int sz_dtype, int64_t n,
                             int g, void* y, int y_dtype, hipStream_t st);
bool dot2_fits(int64_t m, int64_t k, int g);
hipError_t launch_w4a16_gemv(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                             const void* scales, const void* zeros, int sz_dtype, int64_t n,
                             int g, void* y, int y_dtype, hipStream_t st);
bool gemv_mfma_fits(int64_t m, int64_t k, int g);
// 2 <= M <= 4 tokens on the 4x4x4 matrix-core shape: K = 4096, g % 32 == 0.
hipError_t launch_w4a16_quad(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                             const void* scales, const void* zeros, int sz_dtype, int64_t n,
                             int g, void* y, int y_dtype, hipStream_t st);
bool quad_fits(int64_t m, int64_t k, int g);
// ws: optional float32 workspace for split K (nullptr or too small: no split).
hipError_t launch_w4a16_gemm(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                             const void* scales, const void* zeros, int sz_dtype, int64_t n,
                             int g, void* y, int y_dtype, void* ws, size_t ws_bytes, hipStream_t st);
bool gemm_fits(int64_t m, int64_t k, int g);
// Bytes of workspace the GEMM uses for split K on this shape (0: it does not
// split); never above kSplitKMaxBytes.
constexpr size_t kSplitKMaxBytes = (size_t)32 << 20;
size_t gemm_workspace_bytes(int64_t m, int64_t k, int64_t n, int g);
// Device address (current device) of the library's static scratch of
// kSplitKMaxBytes, for callers that cannot allocate.
hipError_t scratch_address(void** out);
hipError_t launch_w4a8_gemv(const int8_t* xq, const float* xs, int64_t m, int64_t k,
                            const uint8_t* packed, const void* scales, const void* zeros,
                            int sz_dtype, int64_t n, int g, void* y, int y_dtype, hipStream_t st);
bool w4a8_gemv_fits(int64_t m, int64_t k, int g);
hipError_t launch_w4a8_gemv_mfma(const int8_t* xq, const float* xs, int64_t m, int64_t k,
                                 const uint8_t* packed, const void* scales, const void* zeros,
                                 int sz_dtype, int64_t n, int g, void* y, int y_dtype,
                                 hipStream_t st);
bool w4a8_gemv_mfma_fits(int64_t m, int64_t k, int g);
// ws: optional float32 workspace for split K (nullptr or too small: no split).
hipError_t launch_w4a8_gemm(const int8_t* xq, const float* xs, int64_t m, int64_t k,
                            const uint8_t* packed, const void* scales, const void* zeros,
                            int sz_dtype, int64_t n, int g, void* y, int y_dtype, void* ws,
                            size_t ws_bytes, hipStream_t st);
bool w4a8_gemm_fits(int64_t m, int64_t k, int g);
// Bytes of workspace the W4A8 GEMM uses for split K on this shape (0: it does
// not split); never above kSplitKMaxBytes.
size_t w4a8_gemm_workspace_bytes(int64_t m, int64_t k, int64_t n, int g);
// y = the sum, in order s = 0 .. S-1, of the float32 partials part + s *
// pstride ([M][N], MN elements each), rounded once to y_dtype.
hipError_t launch_splitk_reduce(const float* part, int S, int64_t mn, int64_t pstride, void* y,
                                int y_dtype, hipStream_t st);
hipError_t launch_w4a8_generic(const int8_t* xq, const float* xs, int64_t m, int64_t k,
                               const uint8_t* packed, const void* scales, const void* zeros,
                               int sz_dtype, int64_t n, int g, void* y, int y_dtype,
                               hipStream_t st);

}  // namespace w4
