// Decode W4A8 GEMV for one to four INT8 tokens: y[m,n] = s_a[m] * sum_g s[n,g] *
// sum_{k in g} xq[m,k] (q[n,k] - zp[n,g]), K of 2048 .. 8192 columns (a
// multiple of 2048), group size 128.  HBM-bound: the packed codes are
// streamed once.
//
// Math ("Hands-on Build Guide: Group-wise INT4 Weight-only Quantization with
// Per-channel Scales", Step 5).  A packed word holds eight codes; its low
// nibbles (codes 0, 2, 4, 6) and high nibbles (codes 1, 3, 5, 7) are each
// four unsigned bytes after one mask, so v_dot4_i32_i8 multiplies them with
// the matching activation bytes, whose even and odd bytes are separated
// once per lane.  Per 32-column run (inside one group) sum xq q and
// zp sum xq are integers below 2^16, so their difference is exact in fp32;
// it is scaled by the group's scale into an fp32 accumulator.
//
// Work layout: as the bf16 dot2 GEMV.  A 256-lane workgroup owns 16 weight
// rows, four per wave; lane l covers the 16-byte chunks l, l + 64, ... of a
// row, so every load instruction reads 1 KB of one row.  The activations
// and the workgroup's scales and zero-points are staged in LDS once; all
// code loads of a wave are issued before any arithmetic.
#include "w4_common.h"
#include "w4_internal.h"

namespace w4 {

namespace {

constexpr int kRowsWave8 = 4;
constexpr int kRowsWg8 = 4 * kRowsWave8;

template <typename TS> struct SZ8;
template <> struct SZ8<_Float16> {
  typedef uint16_t T;
  __device__ static float f(T v) { return (float)__builtin_bit_cast(_Float16, v); }
};
template <> struct SZ8<float> {
  typedef uint32_t T;
  __device__ static float f(T v) { return __uint_as_float(v); }
};

// Sum over the 64 lanes of a wave, result valid in lane 63 (DPP row ops).
__device__ __forceinline__ float wave_sum63(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x111, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x112, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x118, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xa, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xc, 0xf, false));
  return v;
}

template <typename TY>
__device__ __forceinline__ void put8(void* y, int64_t i, float v) {
  if constexpr (sizeof(TY) == 4) {
    ((float*)y)[i] = v;
  } else {
    ((uint16_t*)y)[i] = (uint16_t)f32_to_bf16_bits(v);
  }
}

}  // namespace

// CH: 16-byte chunks per lane and row (K = 2048 CH); MT: tokens (1..4).
template <typename TS, typename TY, int CH, int MT>
__global__ __launch_bounds__(256) void k_w4a8_dot4(
    const int8_t* __restrict__ xq, const float* __restrict__ xscale, int64_t K,
    const uint8_t* __restrict__ packed, const void* __restrict__ scales,
    const void* __restrict__ zeros, int64_t N, int g, void* __restrict__ y) {
  typedef typename SZ8<TS>::T R;
  // LDS: activations [MT][K] int8 (MT K/16 groups of 16 bytes, rounded up to
  // the staging lanes), then the (s, zp) tile of the workgroup's rows.
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  constexpr int XPER = (MT * CH * 2048 / 16 + 255) / 256;
  u32x4* x_l = (u32x4*)lds;
  float2* sz_l = (float2*)(lds + XPER * 256 * 16);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t n0 = (int64_t)blockIdx.x * kRowsWg8;

  // ---- staging loads (activations, scale / zero-point tile) ---------------
  const int xgroups = MT * (int)(K / 16);
  u32x4 xv[XPER];
#pragma unroll
  for (int r = 0; r < XPER; ++r) {
    const int i = tid + 256 * r;
    xv[r] = ((const u32x4*)xq)[i < xgroups ? i : xgroups - 1];
  }
  // scale / zero-point tile: 16 rows x NG groups, CH elements per thread
  constexpr int NG = 16 * CH;  // groups per row (group size 128)
  R sv[CH], zv[CH];
#pragma unroll
  for (int r = 0; r < CH; ++r) {
    const int e = tid + 256 * r;
    const int rr = e / NG, q = e - rr * NG;
    const int64_t row = (n0 + rr) < N ? (n0 + rr) : (N - 1);
    sv[r] = ((const R*)scales)[row * NG + q];
    zv[r] = ((const R*)zeros)[row * NG + q];
  }

  // ---- codes of the wave's rows: 4 x CH 16-byte loads per lane ------------
  u32x4 wq[kRowsWave8][CH];
#pragma unroll
  for (int r = 0; r < kRowsWave8; ++r) {
    int64_t n = n0 + wave * kRowsWave8 + r;
    n = n < N ? n : N - 1;
    const u32x4* row = (const u32x4*)(packed + n * (K / 2));
#pragma unroll
    for (int c = 0; c < CH; ++c) wq[r][c] = __builtin_nontemporal_load(row + lane + 64 * c);
  }
  float sa[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) sa[m] = xscale[m];
  __builtin_amdgcn_sched_barrier(0);

  // ---- LDS stores, barrier -------------------------------------------------
#pragma unroll
  for (int r = 0; r < XPER; ++r) x_l[tid + 256 * r] = xv[r];
#pragma unroll
  for (int r = 0; r < CH; ++r) sz_l[tid + 256 * r] = float2{SZ8<TS>::f(sv[r]), -SZ8<TS>::f(zv[r])};
  __syncthreads();

  // ---- the lane's activations: even / odd bytes of each 8-byte word; sums -
  uint32_t xe[MT][CH][4], xo[MT][CH][4];
  float xs[MT][CH];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    // columns 32 (lane + 64 c) .. + 31 = bytes of 16-byte groups 2 (lane + 64 c), + 1
    const u32x4 a = x_l[m * (K / 16) + 2 * (lane + 64 * c)];
    const u32x4 b = x_l[m * (K / 16) + 2 * (lane + 64 * c) + 1];
    const uint32_t wds[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    int s = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t lo = wds[2 * t], hi = wds[2 * t + 1];  // x[8t .. 8t+3], x[8t+4 .. 8t+7]
      xe[m][c][t] = __builtin_amdgcn_perm(hi, lo, 0x06040200u);  // x0 x2 x4 x6
      xo[m][c][t] = __builtin_amdgcn_perm(hi, lo, 0x07050301u);  // x1 x3 x5 x7
      s = __builtin_amdgcn_sdot4((int)lo, 0x01010101, s, false);
      s = __builtin_amdgcn_sdot4((int)hi, 0x01010101, s, false);
    }
    xs[m][c] = (float)s;
  }
  int gq[CH];  // group of the lane's chunk c
#pragma unroll
  for (int c = 0; c < CH; ++c) gq[c] = (lane + 64 * c) >> 2;

  // ---- rows -------------------------------------------------------------------
#pragma unroll
  for (int r = 0; r < kRowsWave8; ++r) {
    const int rr = wave * kRowsWave8 + r;
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const uint32_t w4[4] = {wq[r][c].x, wq[r][c].y, wq[r][c].z, wq[r][c].w};
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        lo[t] = w4[t] & 0x0f0f0f0fu;
        hi[t] = (w4[t] >> 4) & 0x0f0f0f0fu;
      }
      // (s, -zp); every term below is an integer under 2^24, exact in fp32
      const float2 sz = sz_l[rr * NG + gq[c]];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        int d0 = 0, d1 = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          d0 = __builtin_amdgcn_sdot4((int)lo[t], (int)xe[m][c][t], d0, false);
          d1 = __builtin_amdgcn_sdot4((int)hi[t], (int)xo[m][c][t], d1, false);
        }
        acc[m] = fmaf(sz.x, fmaf(sz.y, xs[m][c], (float)(d0 + d1)), acc[m]);
      }
    }
    const int64_t n = n0 + rr;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float tot = wave_sum63(acc[m]);
      if (lane == 63 && n < N) put8<TY>(y, (int64_t)m * N + n, sa[m] * tot);
    }
  }
}

bool w4a8_gemv_fits(int64_t m, int64_t k, int g) {
  return m >= 1 && m <= 4 && k % 2048 == 0 && k <= 8192 && g == 128;
}

template <typename TS, typename TY, int MT>
static void w4a8_gemv_go(const int8_t* xq, const float* xs, int64_t k, const uint8_t* packed,
                         const void* scales, const void* zeros, int64_t n, int g, void* y,
                         hipStream_t st) {
  const dim3 grid((unsigned)((n + kRowsWg8 - 1) / kRowsWg8));
  const int ch = (int)(k / 2048);
  const size_t lds = (size_t)((MT * ch * 2048 / 16 + 255) / 256) * 256 * 16 + (size_t)ch * 256 * 8;
  switch (ch) {
    case 1: k_w4a8_dot4<TS, TY, 1, MT><<<grid, 256, lds, st>>>(xq, xs, k, packed, scales, zeros, n, g, y); break;
    case 2: k_w4a8_dot4<TS, TY, 2, MT><<<grid, 256, lds, st>>>(xq, xs, k, packed, scales, zeros, n, g, y); break;
    case 3: k_w4a8_dot4<TS, TY, 3, MT><<<grid, 256, lds, st>>>(xq, xs, k, packed, scales, zeros, n, g, y); break;
    default: k_w4a8_dot4<TS, TY, 4, MT><<<grid, 256, lds, st>>>(xq, xs, k, packed, scales, zeros, n, g, y); break;
  }
}

template <typename TS, typename TY>
static void w4a8_gemv_pick(const int8_t* xq, const float* xs, int64_t m, int64_t k,
                           const uint8_t* packed, const void* scales, const void* zeros, int64_t n,
                           int g, void* y, hipStream_t st) {
  if (m == 1) w4a8_gemv_go<TS, TY, 1>(xq, xs, k, packed, scales, zeros, n, g, y, st);
  else if (m == 2) w4a8_gemv_go<TS, TY, 2>(xq, xs, k, packed, scales, zeros, n, g, y, st);
  else if (m == 3) w4a8_gemv_go<TS, TY, 3>(xq, xs, k, packed, scales, zeros, n, g, y, st);
  else w4a8_gemv_go<TS, TY, 4>(xq, xs, k, packed, scales, zeros, n, g, y, st);
}

hipError_t launch_w4a8_gemv(const int8_t* xq, const float* xs, int64_t m, int64_t k,
                            const uint8_t* packed, const void* scales, const void* zeros,
                            int sz_dtype, int64_t n, int g, void* y, int y_dtype, hipStream_t st) {
  if (sz_dtype == W4_F16) {
    if (y_dtype == W4_F32) w4a8_gemv_pick<_Float16, float>(xq, xs, m, k, packed, scales, zeros, n, g, y, st);
    else w4a8_gemv_pick<_Float16, __bf16>(xq, xs, m, k, packed, scales, zeros, n, g, y, st);
  } else {
    if (y_dtype == W4_F32) w4a8_gemv_pick<float, float>(xq, xs, m, k, packed, scales, zeros, n, g, y, st);
    else w4a8_gemv_pick<float, __bf16>(xq, xs, m, k, packed, scales, zeros, n, g, y, st);
  }
  return hipGetLastError();
}

}  // namespace w4
