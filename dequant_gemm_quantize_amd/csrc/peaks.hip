// Measurement kernels for the roofline denominators (libw4peaks.so): what
// this GPU sustains for a plain streaming read and for back-to-back matrix
// instructions, measured beside the INT4 kernels.  They compute nothing of
// the quantization method.
//
//  - k_stream_read: every 16-byte chunk of a buffer read once with the
//    access pattern of the decode kernels (each wavefront load instruction
//    covers 1 KB contiguous, all of a lane's loads issued before any use,
//    non-temporal), xor-folded so the loads stay live.
//  - k_mfma_loop_bf16 / k_mfma_loop_i8: each wavefront issues `iters` rounds
//    of four independent v_mfma_f32_32x32x16_bf16 (32768 flops each) or
//    v_mfma_i32_32x32x32_i8 (65536 ops each) chains on operands loaded from
//    memory (their bit patterns set the power draw, hence the clock).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/w4_peaks.h"
#include "w4_common.h"

namespace w4 {
namespace {

template <int L>
__global__ __launch_bounds__(256) void k_stream_read(const u32x4* __restrict__ src, int64_t nchunks,
                                                     uint32_t* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * (256 * L) + threadIdx.x;
  u32x4 v[L];
#pragma unroll
  for (int j = 0; j < L; ++j) {
    const int64_t c = base + 256 * j;
    v[j] = c < nchunks ? ldg_nt(src + c) : u32x4{0u, 0u, 0u, 0u};
  }
  u32x4 a = v[0];
#pragma unroll
  for (int j = 1; j < L; ++j) a ^= v[j];
  const uint32_t r = a.x ^ a.y ^ a.z ^ a.w;
  if (r == 0x9e3779b9u) sink[0] = r;  // data-dependent store: keeps every load
}

__global__ __launch_bounds__(256) void k_mfma_loop_bf16(const u32x4* __restrict__ operands, int iters,
                                                        float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const bf16x8 a = __builtin_bit_cast(bf16x8, operands[lane]);
  const bf16x8 b = __builtin_bit_cast(bf16x8, operands[64 + lane]);
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += (c0[r] + c1[r]) + (c2[r] + c3[r]);
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void k_mfma_loop_i8(const u32x4* __restrict__ operands, int iters,
                                                      int32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const i32x4 a = __builtin_bit_cast(i32x4, operands[lane]);
  const i32x4 b = __builtin_bit_cast(i32x4, operands[64 + lane]);
  i32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
  }
  int32_t s = 0;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += (c0[r] + c1[r]) + (c2[r] + c3[r]);
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace w4

extern "C" {

int w4_peak_stream_read(const void* src, int64_t bytes, int32_t loads_per_lane, uint32_t* sink,
                        hipStream_t stream) {
  if (src == nullptr || sink == nullptr || !w4::aligned16(src)) return W4_PEAK_EINVAL;
  if (bytes <= 0 || bytes % 16 != 0 || bytes > ((int64_t)1 << 40)) return W4_PEAK_EINVAL;
  if (loads_per_lane != 2 && loads_per_lane != 4 && loads_per_lane != 8 && loads_per_lane != 16 &&
      loads_per_lane != 32)
    return W4_PEAK_EINVAL;
  const int64_t nchunks = bytes / 16;
  const int64_t per_block = 256 * (int64_t)loads_per_lane;
  const int64_t blocks = (nchunks + per_block - 1) / per_block;
  if (blocks > 0x7fffffff) return W4_PEAK_EINVAL;
  const dim3 grid((unsigned)blocks);
  const w4::u32x4* s = (const w4::u32x4*)src;
  switch (loads_per_lane) {
    case 2: w4::k_stream_read<2><<<grid, 256, 0, stream>>>(s, nchunks, sink); break;
    case 4: w4::k_stream_read<4><<<grid, 256, 0, stream>>>(s, nchunks, sink); break;
    case 8: w4::k_stream_read<8><<<grid, 256, 0, stream>>>(s, nchunks, sink); break;
    case 16: w4::k_stream_read<16><<<grid, 256, 0, stream>>>(s, nchunks, sink); break;
    default: w4::k_stream_read<32><<<grid, 256, 0, stream>>>(s, nchunks, sink); break;
  }
  return hipGetLastError() == hipSuccess ? W4_PEAK_OK : W4_PEAK_EHIP;
}

int w4_peak_mfma_loop(int32_t kind, const void* operands, int32_t blocks, int32_t iters, void* out,
                      hipStream_t stream) {
  if (operands == nullptr || out == nullptr || !w4::aligned16(operands) || !w4::aligned16(out))
    return W4_PEAK_EINVAL;
  if (blocks < 1 || blocks > (1 << 20) || iters < 1) return W4_PEAK_EINVAL;
  const w4::u32x4* o = (const w4::u32x4*)operands;
  if (kind == W4_PEAK_BF16)
    w4::k_mfma_loop_bf16<<<blocks, 256, 0, stream>>>(o, iters, (float*)out);
  else if (kind == W4_PEAK_I8)
    w4::k_mfma_loop_i8<<<blocks, 256, 0, stream>>>(o, iters, (int32_t*)out);
  else
    return W4_PEAK_EINVAL;
  return hipGetLastError() == hipSuccess ? W4_PEAK_OK : W4_PEAK_EHIP;
}

}  // extern "C"
