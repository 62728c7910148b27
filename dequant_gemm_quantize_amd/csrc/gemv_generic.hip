// General-purpose fused dequantize-GEMV kernels (any M, any g % 32 == 0,
// fp32 or bf16 activations).  They are the path for fp32 activations and for
// shapes the specialised decode/prefill kernels do not take.
//
// Layout of the work: one wave per output row n, four rows per 256-lane
// block; each lane walks the row in 32-column chunks (16 bytes of packed
// codes, always inside one group since g % 32 == 0).  Per chunk and token
// the lane forms dot = sum q*x and xs = sum x in float32 and adds
// scale * (dot - zp * xs), which is sum x * (q - zp) * scale regrouped
// ("From Scratch: Building a GPTQ INT4 Quantizer in Pure Python", Step 4,
// inside the product of "Build a GPTQ INT4 Quantization Engine in
// Python/NumPy", Step 5).  blockIdx.y selects a slice of up to 8 tokens.
#include "w4_common.h"
#include "w4_internal.h"

namespace w4 {

template <typename TX> struct LoadX32;
// 32 consecutive activations of one token, widened to float32.
template <> struct LoadX32<__bf16> {
  __device__ static void run(const void* x, int64_t off, float (&v)[32]) {
    const u32x4* p = (const u32x4*)((const uint16_t*)x + off);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 a = p[j];
      v[8 * j + 0] = bf16_lo(a.x); v[8 * j + 1] = bf16_hi(a.x);
      v[8 * j + 2] = bf16_lo(a.y); v[8 * j + 3] = bf16_hi(a.y);
      v[8 * j + 4] = bf16_lo(a.z); v[8 * j + 5] = bf16_hi(a.z);
      v[8 * j + 6] = bf16_lo(a.w); v[8 * j + 7] = bf16_hi(a.w);
    }
  }
};
template <> struct LoadX32<float> {
  __device__ static void run(const void* x, int64_t off, float (&v)[32]) {
    const f32x4* p = (const f32x4*)((const float*)x + off);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      f32x4 a = p[j];
      v[4 * j + 0] = a.x; v[4 * j + 1] = a.y; v[4 * j + 2] = a.z; v[4 * j + 3] = a.w;
    }
  }
};

template <typename TY>
__device__ __forceinline__ void store_y(void* y, int64_t i, float v) {
  if constexpr (sizeof(TY) == 4) {
    ((float*)y)[i] = v;
  } else {
    ((uint16_t*)y)[i] = (uint16_t)f32_to_bf16_bits(v);
  }
}

constexpr int kMT = 8;  // tokens per block slice

template <typename TX, typename TS, typename TY>
__global__ __launch_bounds__(256) void k_gemv_w4a16_generic(
    const void* __restrict__ x, int64_t M, int64_t K, const uint8_t* __restrict__ packed,
    const void* __restrict__ scales, const void* __restrict__ zeros, int64_t N, int g,
    void* __restrict__ y) {
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (n >= N) return;  // uniform per wave
  for (int64_t m0 = (int64_t)blockIdx.y * kMT; m0 < M; m0 += (int64_t)gridDim.y * kMT) {
  const int mt = (int)((M - m0) < kMT ? (M - m0) : kMT);
  const int64_t nch = K / 32;
  const int64_t ng = K / g;
  const u32x4* prow = (const u32x4*)(packed + n * (K / 2));
  float acc[kMT];
#pragma unroll
  for (int t = 0; t < kMT; ++t) acc[t] = 0.0f;
  for (int64_t c = lane; c < nch; c += kWave) {
    const u32x4 pw = prow[c];
    const int64_t gi = n * ng + (c * 32) / g;
    const float s = ScaleT<TS>::load(scales, gi);
    const float zp = ScaleT<TS>::load(zeros, gi);
    float q[32];
    const uint32_t w4[4] = {pw.x, pw.y, pw.z, pw.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) q[8 * j + i] = (float)((w4[j] >> (4 * i)) & 15u);
#pragma unroll
    for (int t = 0; t < kMT; ++t) {
      if (t < mt) {
        float xv[32];
        LoadX32<TX>::run(x, (m0 + t) * K + c * 32, xv);
        float dot = 0.0f, xs = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          dot = fmaf(q[i], xv[i], dot);
          xs += xv[i];
        }
        acc[t] = fmaf(s, dot - zp * xs, acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kMT; ++t) {
    if (t < mt) {
      const float r = wave_sum<kWave>(acc[t]);
      if (lane == 0) store_y<TY>(y, (m0 + t) * N + n, r);
    }
  }
  }
}

// INT8-activation variant ("Hands-on Build Guide: Group-wise INT4
// Weight-only Quantization with Per-channel Scales", Step 5): per chunk the
// integer sum xq * (q - zp) is exact in int32 (4-way int8 dot products), then
// scaled by the group scale in float32; the token scale is applied once.
template <typename TS, typename TY>
__global__ __launch_bounds__(256) void k_gemv_w4a8_generic(
    const int8_t* __restrict__ xq, const float* __restrict__ xscale, int64_t M, int64_t K,
    const uint8_t* __restrict__ packed, const void* __restrict__ scales,
    const void* __restrict__ zeros, int64_t N, int g, void* __restrict__ y) {
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (n >= N) return;
  for (int64_t m0 = (int64_t)blockIdx.y * kMT; m0 < M; m0 += (int64_t)gridDim.y * kMT) {
  const int mt = (int)((M - m0) < kMT ? (M - m0) : kMT);
  const int64_t nch = K / 32;
  const int64_t ng = K / g;
  const u32x4* prow = (const u32x4*)(packed + n * (K / 2));
  float acc[kMT];
#pragma unroll
  for (int t = 0; t < kMT; ++t) acc[t] = 0.0f;
  for (int64_t c = lane; c < nch; c += kWave) {
    const u32x4 pw = prow[c];
    const int64_t gi = n * ng + (c * 32) / g;
    const float s = ScaleT<TS>::load(scales, gi);
    const int zp = (int)ScaleT<TS>::load(zeros, gi);
    // codes of the even / odd columns of each 8-column word, one per byte
    const uint32_t w4[4] = {pw.x, pw.y, pw.z, pw.w};
    uint32_t qe[4], qo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qe[j] = w4[j] & 0x0f0f0f0fu;
      qo[j] = (w4[j] >> 4) & 0x0f0f0f0fu;
    }
#pragma unroll
    for (int t = 0; t < kMT; ++t) {
      if (t < mt) {
        const u32x4* xp = (const u32x4*)(xq + (m0 + t) * K + c * 32);
        const u32x4 xa = xp[0], xb = xp[1];
        const uint32_t xw[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
        int dot = 0, xs = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t lo = xw[2 * j], hi = xw[2 * j + 1];
          // bytes (x0, x2, x4, x6) and (x1, x3, x5, x7) of the 8 activations
          const uint32_t xe = __builtin_amdgcn_perm(hi, lo, 0x06040200u);
          const uint32_t xo = __builtin_amdgcn_perm(hi, lo, 0x07050301u);
          dot = __builtin_amdgcn_sdot4((int)qe[j], (int)xe, dot, false);
          dot = __builtin_amdgcn_sdot4((int)qo[j], (int)xo, dot, false);
          xs = __builtin_amdgcn_sdot4((int)lo, 0x01010101, xs, false);
          xs = __builtin_amdgcn_sdot4((int)hi, 0x01010101, xs, false);
        }
        acc[t] = fmaf(s, (float)(dot - zp * xs), acc[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kMT; ++t) {
    if (t < mt) {
      const float r = wave_sum<kWave>(acc[t]);
      if (lane == 0) store_y<TY>(y, (m0 + t) * N + n, r * xscale[m0 + t]);
    }
  }
  }
}

static int64_t token_slices(int64_t M) {
  const int64_t s = (M + kMT - 1) / kMT;
  return s < 65535 ? s : 65535;
}

template <typename TX, typename TS>
static hipError_t gemv16(const void* x, int64_t M, int64_t K, const uint8_t* packed,
                         const void* scales, const void* zeros, int64_t N, int g, void* y,
                         int y_dtype, hipStream_t st) {
  const dim3 grid((unsigned)((N + 3) / 4), (unsigned)token_slices(M));
  if (y_dtype == W4_F32)
    k_gemv_w4a16_generic<TX, TS, float><<<grid, 256, 0, st>>>(x, M, K, packed, scales, zeros, N,
                                                              g, y);
  else
    k_gemv_w4a16_generic<TX, TS, __bf16><<<grid, 256, 0, st>>>(x, M, K, packed, scales, zeros,
                                                               N, g, y);
  return hipGetLastError();
}

hipError_t launch_w4a16_generic(const void* x, int x_dtype, int64_t m, int64_t k,
                                const uint8_t* packed, const void* scales, const void* zeros,
                                int sz_dtype, int64_t n, int g, void* y, int y_dtype,
                                hipStream_t st) {
  const bool xb = (x_dtype == W4_BF16), sh = (sz_dtype == W4_F16);
  if (xb && sh) return gemv16<__bf16, _Float16>(x, m, k, packed, scales, zeros, n, g, y, y_dtype, st);
  if (xb) return gemv16<__bf16, float>(x, m, k, packed, scales, zeros, n, g, y, y_dtype, st);
  if (sh) return gemv16<float, _Float16>(x, m, k, packed, scales, zeros, n, g, y, y_dtype, st);
  return gemv16<float, float>(x, m, k, packed, scales, zeros, n, g, y, y_dtype, st);
}

hipError_t launch_w4a8_generic(const int8_t* xq, const float* xs, int64_t m, int64_t k,
                               const uint8_t* packed, const void* scales, const void* zeros,
                               int sz_dtype, int64_t n, int g, void* y, int y_dtype,
                               hipStream_t st) {
  const dim3 grid((unsigned)((n + 3) / 4), (unsigned)token_slices(m));
  const bool sh = (sz_dtype == W4_F16);
  if (sh && y_dtype == W4_F32)
    k_gemv_w4a8_generic<_Float16, float><<<grid, 256, 0, st>>>(xq, xs, m, k, packed, scales, zeros, n, g, y);
  else if (sh)
    k_gemv_w4a8_generic<_Float16, __bf16><<<grid, 256, 0, st>>>(xq, xs, m, k, packed, scales, zeros, n, g, y);
  else if (y_dtype == W4_F32)
    k_gemv_w4a8_generic<float, float><<<grid, 256, 0, st>>>(xq, xs, m, k, packed, scales, zeros, n, g, y);
  else
    k_gemv_w4a8_generic<float, __bf16><<<grid, 256, 0, st>>>(xq, xs, m, k, packed, scales, zeros, n, g, y);
  return hipGetLastError();
}

}  // namespace w4
