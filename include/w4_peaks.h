/*
 * w4_peaks.h -- measurement kernels of libw4peaks.so: the streaming-read and
 * matrix-instruction rates that the roofline fractions of libw4 are set
 * beside.  They are not part of the quantization method.  Same conventions
 * as w4.h: device pointers, asynchronous on `stream`, the caller owns every
 * buffer, invalid arguments are rejected before any HIP call.
 */
#ifndef W4_PEAKS_H_
#define W4_PEAKS_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { W4_PEAK_OK = 0, W4_PEAK_EINVAL = -1, W4_PEAK_EHIP = -3 };
enum { W4_PEAK_BF16 = 0, W4_PEAK_I8 = 1 };

/*
 * w4_peak_stream_read -- reads `bytes` (a multiple of 16, > 0) of `src`
 * (16-byte aligned) once.  Workgroups of 256 lanes; each lane issues
 * loads_per_lane (2, 4, 8, 16 or 32) 16-byte non-temporal loads, each wavefront load
 * instruction covering 1 KB contiguous -- the pattern of the decode kernels
 * (8 loads per lane reproduces their geometry on the [11008, 4096] weight).
 * The loaded words are xor-folded; `sink` (4 bytes) is written only when the
 * fold equals one fixed value, so it is almost never written.  Bytes moved:
 * `bytes` read, nothing written.
 */
int w4_peak_stream_read(const void* src, int64_t bytes, int32_t loads_per_lane, uint32_t* sink,
                        hipStream_t stream);

/*
 * w4_peak_mfma_loop -- `blocks` workgroups of four wavefronts; each wavefront
 * runs `iters` rounds of four independent accumulation chains of
 * v_mfma_f32_32x32x16_bf16 (kind W4_PEAK_BF16: 32768 flops per instruction)
 * or v_mfma_i32_32x32x32_i8 (kind W4_PEAK_I8: 65536 ops per instruction).
 * Operands: 128 16-byte values at `operands` (lane l takes values l and
 * 64 + l).  `out`: one float32 or int32 per lane (blocks * 256 values) with
 * the folded accumulators.  Work per launch: blocks * 4 * iters * 4 *
 * (32768 or 65536).
 */
int w4_peak_mfma_loop(int32_t kind, const void* operands, int32_t blocks, int32_t iters, void* out,
                      hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* W4_PEAKS_H_ */
