/*
 * w4.h -- C ABI of libw4: group-wise asymmetric INT4 weight quantization and
 * the dequantize-matmul that consumes it, for AMD Instinct MI355X (gfx950).
 *
 * Method (martinuke0.github.io posts):
 *   [P1] "Hands-on Build Guide: Group-wise INT4 Weight-only Quantization with
 *        Per-channel Scales"
 *   [P2] "From-scratch INT4 Weight-only Quantizer with Per-group Scales and
 *        Zero-points for LLMs"
 *   [P3] "Building a From-Scratch Group-Wise INT4 Quantization Layer for
 *        LLaMA Weights"
 *   [P4] "Build a GPTQ INT4 Quantization Engine in Python/NumPy"
 *   [P5] "From Scratch: Building a GPTQ INT4 Quantizer in Pure Python"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Shapes: N = out_features, K = in_features, M = tokens, g = group size.
 *    W is [N, K] ("nn.Linear" layout), x is [M, K], y is [M, N].  Every
 *    tensor is dense, row-major, with no padding between rows.
 *  - A group is a run of g consecutive elements of one row of W (along K).
 *    Requirements: g % 32 == 0, K % g == 0.  scales and zeros are [N, K/g].
 *  - packed is uint8 [N, K/2]; byte j of row n holds the code of column 2j in
 *    its low nibble and of column 2j+1 in its high nibble ([P4] Step 4).
 *  - zeros are stored in the same dtype as scales and hold the integers
 *    0..15 exactly (+0.0 for zero).
 *  - Pointers are device pointers (hipMalloc'd or equivalent) and must be
 *    16-byte aligned.  The caller owns every buffer; the library never
 *    allocates, frees or synchronizes.  Work is enqueued on `stream` (0 = the
 *    null stream) and is asynchronous: outputs are valid once the stream has
 *    reached that point.  Calls on one stream are ordered; calls on different
 *    streams that write the same buffer race.
 *  - Errors: arguments are validated before any HIP call; an invalid call
 *    returns W4_EINVAL and enqueues nothing.  A failed launch returns W4_EHIP.
 *    w4_last_error() gives a message for the last failure on the calling
 *    thread.  No C++ exception crosses this interface.
 *  - M == 0 or N == 0 is a valid empty call: it returns W4_OK and enqueues
 *    nothing.  K must be > 0.
 *  - Size limits (W4_EINVAL beyond them): K <= 2^23; N*K, M*K and M*N each
 *    <= 2^36 elements; M < 2^31 (M < 2^24 for quantize_act_int8).
 *  - Inputs must be finite; NaN or Inf inputs, and group ranges that overflow
 *    the scale dtype (fp16 scales: (max - min) / 15 > 65504), give unspecified
 *    (but memory-safe) results.
 */
#ifndef W4_H_
#define W4_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types (the `*_dtype` arguments). */
enum w4_dtype { W4_F32 = 0, W4_F16 = 1, W4_BF16 = 2 };

/* Return codes. */
enum w4_status {
  W4_OK = 0,
  W4_EINVAL = -1,       /* bad argument: null/misaligned pointer, bad shape or dtype */
  W4_EUNSUPPORTED = -2, /* valid request this build does not implement */
  W4_EHIP = -3          /* the HIP runtime reported an error */
};

/*
 * quantize_pack_int4 -- group-wise asymmetric INT4 round-to-nearest + pack.
 *
 * For each group G of W ([P2] Architecture Overview and Steps 5-6;
 * [P5] Step 2), in IEEE float32 with round-to-nearest-even:
 *   mn = min(G), mx = max(G)
 *   scale  = (mx - mn) / 15, rounded to sz_dtype; a stored 0 becomes 1
 *   zp     = clamp(rint(-mn / scale), 0, 15)   (with the stored scale)
 *   q(w)   = clamp(rint(w / scale + zp), 0, 15)  (rint: ties to even)
 * and the codes are packed two per byte, even column in the low nibble.
 *
 *   w        [N, K] input weights, w_dtype W4_F32 or W4_BF16
 *   packed   [N, K/2] uint8 output
 *   scales   [N, K/g] output, sz_dtype W4_F32 or W4_F16
 *   zeros    [N, K/g] output, same dtype as scales
 * The outputs are bit-for-bit those of the definition above.
 */
int quantize_pack_int4(const void* w, int w_dtype, int64_t n, int64_t k, int32_t group_size,
                       uint8_t* packed, void* scales, void* zeros, int sz_dtype,
                       hipStream_t stream);

/*
 * quantize_pack_int4_sym -- group-wise symmetric INT4 round-to-nearest + pack.
 *
 * For each group G of W ([P4] Step 2 for scale and codes, Step 4 for the
 * +8 storage offset), in IEEE float32 with round-to-nearest-even:
 *   amax   = max(|G|)
 *   scale  = amax / 7, rounded to sz_dtype; a stored 0 becomes 1
 *   q(w)   = clamp(rint(w / scale), -8, 7) + 8   (with the stored scale;
 *            the offset is added after rounding)
 * and the codes are packed two per byte, even column in the low nibble.
 * Every zero-point is 8, and zeros[] is written with 8, so dequant_int4,
 * w4a16_matmul and w4a8_matmul take the three outputs unchanged and compute
 * (q - 8) * scale.  Arguments, layout, limits and errors are those of
 * quantize_pack_int4.  The outputs are bit-for-bit those of the definition.
 */
int quantize_pack_int4_sym(const void* w, int w_dtype, int64_t n, int64_t k, int32_t group_size,
                           uint8_t* packed, void* scales, void* zeros, int sz_dtype,
                           hipStream_t stream);

/*
 * quantize_pack_int4_sym_percentile / quantize_pack_int4_sym_mse -- the
 * symmetric format with a calibrated scale per group ([P3] Step 4's
 * range-clipping calibrators); the codes are then those of
 * quantize_pack_int4_sym with the stored scale, zeros[] is written with 8.
 *
 * Both follow the PyTorch calls of that step on the float32 group.
 * percentile: range = torch.quantile(|G|, p / 100) for 0 < p <= 100, in
 *   float32: with a = sorted |G|, rank = fl32(fl32(p / 100) * (g - 1)),
 *   i0 = floor(rank), i1 = ceil(rank), f = rank - i0, d = a[i1] - a[i0]:
 *   range = fma(f, d, a[i0]) if f < 1/2, else fma(f - 1, d, a[i1]) (one
 *   rounding each); scale = range / 7 (p = 100 gives quantize_pack_int4_sym
 *   exactly).
 * mse: `candidates` = n (2 .. 65536) steps torch.linspace(lo, hi, n) with
 *   lo = min|G|, hi = max|G|: d = (hi - lo) / (n - 1), c_i = fma(d, i, lo)
 *   for i < n / 2 and fma(-d, n - 1 - i, hi) otherwise (float32); a step
 *   below 1e-10 is skipped; for the others q = clamp(rint(w / c), -7, 7)
 *   (float32 division) and E(c) = (sum over G, in column order, of
 *   (q c - w)^2) / g in float32; the step is the first c with the least E,
 *   or 1e-8 when none qualifies.  The cost is about 10 g n float32
 *   operations per group.
 * Both: group_size <= 1024 (W4_EINVAL above); otherwise arguments, layout,
 * limits and errors as quantize_pack_int4.  The outputs are bit-for-bit
 * those of the definitions above.
 */
int quantize_pack_int4_sym_percentile(const void* w, int w_dtype, int64_t n, int64_t k,
                                      int32_t group_size, double percentile, uint8_t* packed,
                                      void* scales, void* zeros, int sz_dtype, hipStream_t stream);
int quantize_pack_int4_sym_mse(const void* w, int w_dtype, int64_t n, int64_t k, int32_t group_size,
                               int32_t candidates, uint8_t* packed, void* scales, void* zeros,
                               int sz_dtype, hipStream_t stream);

/*
 * dequant_int4 -- w_out[n, k] = (q[n, k] - zp[n, k/g]) * scale[n, k/g]
 * ([P5] Step 4), computed as one float32 product of the exact integer
 * difference and the scale, then rounded (nearest-even) to out_dtype
 * (W4_F32, W4_F16 or W4_BF16).  w_out is [N, K].  Bit-exact; this is the
 * unfused form, used to check and compare the fused matmuls.
 */
int dequant_int4(const uint8_t* packed, const void* scales, const void* zeros, int sz_dtype,
                 int64_t n, int64_t k, int32_t group_size, void* w_out, int out_dtype,
                 hipStream_t stream);

/*
 * quantize_act_int8 -- per-token dynamic INT8 activations ([P1]
 * Architecture Overview, Step 3), in IEEE float32:
 *   x_scale[m] = max(max_k |x[m, k]|, 1e-8) / 127
 *   xq[m, k]   = clamp(rint(x[m, k] / x_scale[m]), -128, 127)
 *   x        [M, K] input, x_dtype W4_F32 or W4_BF16; K % 8 == 0
 *   xq       [M, K] int8 output;  x_scale [M] float32 output (4-byte aligned).
 *   M < 2^24 tokens (W4_EINVAL otherwise).
 * Bit-exact.
 */
int quantize_act_int8(const void* x, int x_dtype, int64_t m, int64_t k, int8_t* xq,
                      float* x_scale, hipStream_t stream);

/*
 * w4a16_matmul -- y = x . dequant(W)^T  ([P3] Step 2; [P4] Step 5), fused:
 * the packed weights are read from memory once per output tile and
 * dequantized in registers/LDS; no dequantized weight matrix is written.
 *   x   [M, K], x_dtype W4_BF16 or W4_F32
 *   y   [M, N], y_dtype W4_BF16 or W4_F32 (float32 accumulation, one
 *       rounding to y_dtype at the end)
 * Accuracy: max|y - y_exact| / max|y_exact| <= 1e-2 for bf16 y and
 * <= 3e-3 for fp32 y, y_exact being the float64 product of the same x and
 * the exactly dequantized weights.  Small M (decode) and large M (prefill)
 * use different kernels; both meet the same bound.  Results are
 * deterministic (no atomics; a fixed reduction order per shape).
 */
int w4a16_matmul(const void* x, int x_dtype, int64_t m, int64_t k, const uint8_t* packed,
                 const void* scales, const void* zeros, int sz_dtype, int64_t n,
                 int32_t group_size, void* y, int y_dtype, hipStream_t stream);

/*
 * w4a16_matmul_workspace_size / w4a16_matmul_ws -- w4a16_matmul with a
 * caller-provided device workspace ([P3] Step 2 and [P4] Step 5; the
 * workspace changes how the product is scheduled, not what it computes).
 *
 * Shapes whose 256 x 128 output tiles fill fewer than half of the GPU's 256
 * compute units (for example the [4096, 11008] down projection at 129 to 512
 * tokens) split K across workgroups: each writes a float32 partial tile to
 * the workspace and a second kernel adds the partials in a fixed order and
 * rounds once to y_dtype.  Results are deterministic and meet the accuracy
 * bound of w4a16_matmul.
 *
 * w4a16_matmul_workspace_size returns the bytes of workspace that let
 * w4a16_matmul_ws split K for this shape: 0 when it would not split (it then
 * behaves as w4a16_matmul), at most 32 MiB.  It depends only on its
 * arguments, enqueues nothing and returns 0 for arguments the other calls
 * reject.
 *
 * w4a16_matmul_ws takes w4a16_matmul's arguments plus `workspace` (device
 * memory, 16-byte aligned, owned by the caller; its contents on entry are
 * ignored and on return unspecified) of `workspace_bytes`.  With
 * workspace_bytes below the queried size, or workspace NULL, it runs
 * exactly as w4a16_matmul.  Calls that overlap on one workspace race.
 * Errors as w4a16_matmul, plus W4_EINVAL for a misaligned workspace.
 */
size_t w4a16_matmul_workspace_size(int64_t m, int64_t k, int64_t n, int32_t group_size,
                                   int x_dtype);
int w4a16_matmul_ws(const void* x, int x_dtype, int64_t m, int64_t k, const uint8_t* packed,
                    const void* scales, const void* zeros, int sz_dtype, int64_t n,
                    int32_t group_size, void* y, int y_dtype, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/*
 * w4a16_matmul_noalloc -- for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): w4a16_matmul_ws with the library's own scratch in place of
 * the caller's workspace, so every shape gets the split-K schedule with no
 * allocation, free or allocating library routine on any call.
 *
 * The scratch is a static device array of 32 MiB (the most any shape's
 * split-K partials take), one per device, held from the library's first use
 * on that device until the process ends.  Every call on a device shares it:
 * calls that overlap on one device (different streams, or different host
 * threads) race and must be ordered by the caller.  Arguments, results,
 * accuracy and errors are those of w4a16_matmul; a shape whose partials
 * would exceed the scratch returns W4_EINVAL (the split plan never asks for
 * more, so no valid call does).
 */
int w4a16_matmul_noalloc(const void* x, int x_dtype, int64_t m, int64_t k, const uint8_t* packed,
                         const void* scales, const void* zeros, int sz_dtype, int64_t n,
                         int32_t group_size, void* y, int y_dtype, hipStream_t stream);

/*
 * w4a8_matmul -- y[m, n] = x_scale[m] * sum_k xq[m, k] * dequant(W)[n, k]
 * ([P1] Architecture Overview, Step 5), with xq/x_scale as produced by
 * quantize_act_int8.  Per group the integer sum of xq * (q - zp) is exact
 * (int32); it is scaled in float32.  y [M, N], y_dtype W4_BF16 or W4_F32.
 * Same accuracy bound and determinism as w4a16_matmul.
 */
int w4a8_matmul(const int8_t* xq, const float* x_scale, int64_t m, int64_t k,
                const uint8_t* packed, const void* scales, const void* zeros, int sz_dtype,
                int64_t n, int32_t group_size, void* y, int y_dtype, hipStream_t stream);

/*
 * w4a8_matmul_workspace_size / w4a8_matmul_ws -- w4a8_matmul with a
 * caller-provided device workspace ([P1] Step 5; the workspace changes how
 * the product is scheduled, not what it computes).
 *
 * Shapes whose output tiles would leave most of the GPU's 256 compute units
 * idle (for example one GPU's 8-way column shard [3584, 8192] of the
 * [28672, 8192] projection at 512 tokens: 56 tiles) split K across
 * workgroups: each writes its token-scaled float32 partial tile to the
 * workspace and a second kernel adds the partials in a fixed order and
 * rounds once to y_dtype.  Results are deterministic and meet the accuracy
 * bound of w4a8_matmul; the integer sums stay exact (a split boundary falls
 * between 128-column K steps, and each step lies inside one group).
 *
 * w4a8_matmul_workspace_size returns the bytes of workspace that let
 * w4a8_matmul_ws split K for this shape: 0 when it would not split (it then
 * behaves as w4a8_matmul), at most 32 MiB.  It depends only on its
 * arguments, enqueues nothing and returns 0 for arguments the other calls
 * reject.
 *
 * w4a8_matmul_ws takes w4a8_matmul's arguments plus `workspace` (device
 * memory, 16-byte aligned, owned by the caller; its contents on entry are
 * ignored and on return unspecified) of `workspace_bytes`.  With
 * workspace_bytes below the queried size, or workspace NULL, it runs
 * exactly as w4a8_matmul.  Calls that overlap on one workspace race.
 * Errors as w4a8_matmul, plus W4_EINVAL for a misaligned workspace.
 */
size_t w4a8_matmul_workspace_size(int64_t m, int64_t k, int64_t n, int32_t group_size);
int w4a8_matmul_ws(const int8_t* xq, const float* x_scale, int64_t m, int64_t k,
                   const uint8_t* packed, const void* scales, const void* zeros, int sz_dtype,
                   int64_t n, int32_t group_size, void* y, int y_dtype, void* workspace,
                   size_t workspace_bytes, hipStream_t stream);

/*
 * GPTQ second-order quantization ([P4] Step 3), in three calls.  Together
 * they produce the packed format above from a weight and calibration rows;
 * every matmul here takes the result.
 *
 * gptq_hessian -- h[K, K] = X^T X / T + 1e-4 * mean(diag(X^T X / T)) * I,
 *   x [T, K] float32 calibration rows (T >= 1), h float64 output (both
 *   triangles written).  Products are exact in float64 and each entry is
 *   summed in row order; the damping term's mean is a fixed-order sum.
 *   1 <= K <= 65536; x and h 16-byte aligned.
 */
int gptq_hessian(const float* x, int64_t t, int64_t k, double* h, hipStream_t stream);

/*
 * gptq_inverse_cholesky -- u[K, K] float64 = the upper-triangular factor U
 *   with U^T U = H^-1 and a positive diagonal (the Cholesky factor of the
 *   inverse, "upper-triangular form"), strictly lower part set to 0.
 *   h [K, K] float64 symmetric positive definite; only its upper triangle
 *   is read, and h is used as workspace: on return its contents are
 *   unspecified.  info: one device int32, set to 0 on success, or to
 *   1 + the index of the first column (the factorization visits columns
 *   from the last to the first) whose pivot was not positive; u is then
 *   unspecified.  The status is decided on the device: the call does not
 *   wait for it.  h, u 16-byte aligned and distinct; 1 <= K <= 65536.
 *   Float64 throughout; the result matches the factor of the exact inverse
 *   to about cond(H) * 1e-16.
 */
int gptq_inverse_cholesky(double* h, int64_t k, double* u, int32_t* info, hipStream_t stream);

/*
 * gptq_quantize_pack_int4 -- the column sweep.  For each row of W [N, K]
 *   (float32, row-major) and each column i from left to right:
 *     when i starts a group, the group's scale and zero-point are computed
 *       from the group's current values with the formulas of
 *       quantize_pack_int4 (symmetric = 0) or quantize_pack_int4_sym
 *       (symmetric != 0, zero-points written as 8);
 *     q_i = the code of w_i with those parameters (the same float32 steps);
 *     e = (w_i - (q_i - zp) * scale) / U[i, i];
 *     w_j -= e * U[i, j] for every j > i.
 *   u is gptq_inverse_cholesky's output.  Outputs packed / scales / zeros
 *   as quantize_pack_int4.  w is working storage: on return column i of
 *   each row holds that row's e for column i.  group_size: 32, 64, or a
 *   multiple of 128 (W4_EINVAL otherwise); 1 <= K <= 65536.  The updates
 *   are applied 128 columns at a time with float32 products, so the values
 *   a code is decided on differ from an exact sweep by rounding; a code or
 *   zero-point can then differ by one where the decision is that close to
 *   a tie.
 */
int gptq_quantize_pack_int4(float* w, const double* u, int64_t n, int64_t k, int32_t group_size,
                            int32_t symmetric, uint8_t* packed, void* scales, void* zeros,
                            int sz_dtype, hipStream_t stream);

/* Static description of a w4_status value (never NULL). */
const char* w4_status_string(int status);

/* Message describing the last failed call on the calling thread ("" if none). */
const char* w4_last_error(void);

/* Library version string, e.g. "w4 0.1.0 gfx950". */
const char* w4_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W4_H_ */
