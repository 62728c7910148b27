// Quantize + pack, dequantize, and per-token INT8 activation kernels.
//
// All three are memory-bound streaming kernels.  Their float32 arithmetic is
// the definition itself -- IEEE division (correctly rounded), rint with ties
// to even, round-to-nearest-even narrowing -- so the outputs are bit-exact.
// Contraction into FMA is switched off in this file: nothing here may fuse.
#include <cmath>

#include "w4_common.h"
#include "w4_internal.h"

#pragma clang fp contract(off)

namespace w4 {

// ---------------------------------------------------------------------------
// Element loads: 8 consecutive elements of chunk c (element index 8c..8c+7).
// ---------------------------------------------------------------------------
template <typename TIn> struct Load8;
template <> struct Load8<float> {  // fp32 input: two 16-byte loads
  __device__ static void run(const void* base, int64_t c, float (&v)[8]) {
    const f32x4* p = (const f32x4*)base + 2 * c;
    f32x4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};
template <> struct Load8<__bf16> {  // bf16 input: one 16-byte load, exact widening
  __device__ static void run(const void* base, int64_t c, float (&v)[8]) {
    u32x4 a = ((const u32x4*)base)[c];
    v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x); v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
    v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z); v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
  }
};

// Scale and zero-point of one group from its range ("From-scratch INT4
// Weight-only Quantizer with Per-group Scales and Zero-points for LLMs",
// Architecture Overview and Step 6): scale = (max - min)/15 rounded to the
// storage type, 0 -> 1; zp = clamp(rint(-min/scale), 0, 15) with that scale.
template <typename TS>
__device__ __forceinline__ void scale_zero(float mn, float mx, TS& s_store, float& s, int& zp) {
  float s32 = (mx - mn) / 15.0f;
  TS st = (TS)s32;
  if (st == (TS)0.0f) st = (TS)1.0f;
  s_store = st;
  s = (float)st;
  float z = rintf(-mn / s);
  z = fminf(fmaxf(z, 0.0f), 15.0f);
  zp = (int)z;
}

// Code of one weight ("From Scratch: Building a GPTQ INT4 Quantizer in Pure
// Python", Step 2): clamp(rint(w/scale + zp), 0, 15).
__device__ __forceinline__ uint32_t code_of(float w, float s, float zpf) {
  float t = rintf(w / s + zpf);
  t = fminf(fmaxf(t, 0.0f), 15.0f);
  return (uint32_t)t;
}

// Eight codes -> one 32-bit word; element i sits in nibble i, so byte j holds
// the even column in its low nibble ("Build a GPTQ INT4 Quantization Engine in
// Python/NumPy", Step 4).
//
// The division is the costly part, so it is skipped where it cannot change
// a code.  t = fma(w, 1/s, zp) differs from the defined fl32(fl32(w/s) + zp)
// by less than 2^-16 whenever |t| < 32 (|w/s| <= |t| + 15; the hardware
// reciprocal (v_rcp_f32, within 1 ulp) and the product add at most 1.5 ulp of
// w/s, the two sums one rounding each).  A code only depends on which side
// of a half-integer in 0.5 .. 14.5 t lies once it is clamped to [0, 15]
// (clamping first changes no code: every t that clamps gives 0 or 15 either
// way).  So unless some clamped t of the word lies within 2^-12 of a
// half-integer -- or 1/s overflows -- rint of the clamped t is the defined
// code; otherwise the word is recomputed with the correctly rounded division.
// r = 1/s from v_rcp_f32.
__device__ __forceinline__ uint32_t pack8(const float* v, float s, float r, float zpf) {
  float c[8];
  float dmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float t = fminf(fmaxf(fmaf(v[i], r, zpf), 0.0f), 15.0f);
    c[i] = rintf(t);
    dmax = fmaxf(dmax, fabsf(t - c[i]));  // exact difference, at most 0.5
  }
  if (!(dmax < 0.5f - 0x1p-12f) || !(r < 3.0e38f)) {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) word |= code_of(v[i], s, zpf) << (4 * i);
    return word;
  }
  // even codes to the bytes of lo, odd codes to the bytes of hi (c is an
  // integer in 0 .. 15, so the byte conversion is exact)
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    lo = __builtin_amdgcn_cvt_pk_u8_f32(c[2 * j], j, lo);
    hi = __builtin_amdgcn_cvt_pk_u8_f32(c[2 * j + 1], j, hi);
  }
  return lo | (hi << 4);
}

// Symmetric variant ("Build a GPTQ INT4 Quantization Engine in
// Python/NumPy", Step 2): scale = absmax / 7 rounded to the storage type,
// 0 -> 1; signed code clamp(rint(w/scale), -8, 7), stored as code + 8
// (Step 4), i.e. a fixed zero-point of 8.  The offset goes onto the rounded
// integer.
template <typename TS>
__device__ __forceinline__ void scale_sym(float amax, TS& s_store, float& s) {
  float s32 = amax / 7.0f;
  TS st = (TS)s32;
  if (st == (TS)0.0f) st = (TS)1.0f;
  s_store = st;
  s = (float)st;
}

__device__ __forceinline__ uint32_t code_sym(float w, float s) {
  float t = rintf(w / s);
  t = fminf(fmaxf(t, -8.0f), 7.0f);
  return (uint32_t)(t + 8.0f);
}

// As pack8, for the symmetric codes.  t = w * (1/s) differs from fl32(w/s)
// by less than 2^-19 wherever |t| <= 8 (1.5 ulp of the product plus the
// division's half ulp), and only the half-integers -7.5 .. 6.5 decide a code
// once t is clamped to [-8, 7] (every t that clamps gives -8 or 7 either
// way).  Words with a clamped t within 2^-12 of a half-integer, or with an
// infinite 1/s, take the correctly rounded division.
__device__ __forceinline__ uint32_t pack8_sym(const float* v, float s, float r) {
  float c[8];
  float dmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float t = fminf(fmaxf(v[i] * r, -8.0f), 7.0f);
    c[i] = rintf(t);
    dmax = fmaxf(dmax, fabsf(t - c[i]));
  }
  if (!(dmax < 0.5f - 0x1p-12f) || !(r < 3.0e38f)) {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) word |= code_sym(v[i], s) << (4 * i);
    return word;
  }
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    lo = __builtin_amdgcn_cvt_pk_u8_f32(c[2 * j] + 8.0f, j, lo);
    hi = __builtin_amdgcn_cvt_pk_u8_f32(c[2 * j + 1] + 8.0f, j, hi);
  }
  return lo | (hi << 4);
}

// Scale, zero-point and reciprocal of a group from its min and max, for
// either variant.
template <typename TS, bool SYM>
__device__ __forceinline__ void group_params(float mn, float mx, TS& st, float& s, float& r,
                                             float& zpf) {
  if constexpr (SYM) {
    scale_sym<TS>(fmaxf(-mn, mx), st, s);
    zpf = 8.0f;
  } else {
    int zp;
    scale_zero<TS>(mn, mx, st, s, zp);
    zpf = (float)zp;
  }
  r = __builtin_amdgcn_rcpf(s);
}

template <bool SYM>
__device__ __forceinline__ uint32_t pack8v(const float* v, float s, float r, float zpf) {
  if constexpr (SYM) return pack8_sym(v, s, r);
  else return pack8(v, s, r, zpf);
}

// ---------------------------------------------------------------------------
// Quantize + pack, groups of g = 32 L elements, L = 1, 2, 4, 8, 16.
// The tensor is treated as a flat run of N*K elements: with K % g == 0 a
// group never crosses a row, and flat group index == row * (K/g) + group.
// Each lane owns pieces of 32 consecutive elements (4 packed words); L
// neighbouring lanes share a group and reduce its min/max with xor
// butterflies, so the per-group work (scale, zero-point, reciprocal) is
// shared by 4 words.  U pieces per lane are loaded up front.
// ---------------------------------------------------------------------------
template <typename TIn, typename TS, int L, int U, bool SYM>
__global__ __launch_bounds__(256) void k_quantize_pack_sub(const void* __restrict__ w,
                                                          int64_t npieces,
                                                          uint32_t* __restrict__ packed,
                                                          TS* __restrict__ scales,
                                                          TS* __restrict__ zeros) {
  const int64_t base = (int64_t)blockIdx.x * (256 * U) + threadIdx.x;
  float v[U][4][8];
  if constexpr (sizeof(TIn) == 2 && U == 1) {
    // bf16: the wave's 4 KB are loaded with consecutive lanes on consecutive
    // 16-byte chunks (fully coalesced), then regrouped through LDS so that
    // lane l holds chunks 4l .. 4l+3.  LDS slots are XOR-swizzled (slot
    // c ^ ((c / 16) mod 4)) so both the stores and the strided reads are free
    // of bank conflicts.
    __shared__ u32x4 stg[4][256];
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t c0 = 4 * ((int64_t)blockIdx.x * 256 + 64 * wv);
    const int64_t nchunks = 4 * npieces;
    u32x4 a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t c = c0 + 64 * j + lane;
      a[j] = c < nchunks ? ((const u32x4*)w)[c] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cl = 64 * j + lane;
      stg[wv][cl ^ ((cl >> 4) & 3)] = a[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cl = 4 * lane + j;
      const u32x4 b = stg[wv][cl ^ ((cl >> 4) & 3)];
      v[0][j][0] = bf16_lo(b.x); v[0][j][1] = bf16_hi(b.x); v[0][j][2] = bf16_lo(b.y); v[0][j][3] = bf16_hi(b.y);
      v[0][j][4] = bf16_lo(b.z); v[0][j][5] = bf16_hi(b.z); v[0][j][6] = bf16_lo(b.w); v[0][j][7] = bf16_hi(b.w);
    }
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t p = base + (int64_t)u * 256;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (p < npieces) {
          Load8<TIn>::run(w, 4 * p + j, v[u][j]);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) v[u][j][i] = 0.0f;
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t p = base + (int64_t)u * 256;
    float mn = v[u][0][0], mx = v[u][0][0];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        mn = fminf(mn, v[u][j][i]);
        mx = fmaxf(mx, v[u][j][i]);
      }
    mn = group_min<L>(mn);
    mx = group_max<L>(mx);
    TS st;
    float s, r, zpf;
    group_params<TS, SYM>(mn, mx, st, s, r, zpf);
    u32x4 words;
    words.x = pack8v<SYM>(v[u][0], s, r, zpf);
    words.y = pack8v<SYM>(v[u][1], s, r, zpf);
    words.z = pack8v<SYM>(v[u][2], s, r, zpf);
    words.w = pack8v<SYM>(v[u][3], s, r, zpf);
    if (p < npieces) {
      ((u32x4*)packed)[p] = words;
      if ((threadIdx.x & (L - 1)) == 0) {
        const int64_t gi = p / L;
        scales[gi] = st;
        zeros[gi] = (TS)zpf;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Quantize + pack, any group size that is a multiple of 8: one wave per
// group, two passes over the group (the second pass reads it from cache).
// ---------------------------------------------------------------------------
template <typename TIn, typename TS, bool SYM>
__global__ __launch_bounds__(256) void k_quantize_pack_wave(const void* __restrict__ w,
                                                           int64_t ngroups, int cpg,
                                                           uint32_t* __restrict__ packed,
                                                           TS* __restrict__ scales,
                                                           TS* __restrict__ zeros) {
  const int64_t grp = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (grp >= ngroups) return;  // uniform per wave
  const int64_t c0 = grp * cpg;
  float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
  for (int c = lane; c < cpg; c += kWave) {
    float v[8];
    Load8<TIn>::run(w, c0 + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      mn = fminf(mn, v[i]);
      mx = fmaxf(mx, v[i]);
    }
  }
  mn = group_min<kWave>(mn);
  mx = group_max<kWave>(mx);
  TS st;
  float s, r, zpf;
  group_params<TS, SYM>(mn, mx, st, s, r, zpf);
  for (int c = lane; c < cpg; c += kWave) {
    float v[8];
    Load8<TIn>::run(w, c0 + c, v);
    packed[c0 + c] = pack8v<SYM>(v, s, r, zpf);
  }
  if (lane == 0) {
    scales[grp] = st;
    zeros[grp] = (TS)zpf;
  }
}

template <typename TIn, typename TS, bool SYM>
static hipError_t launch_qp(const void* w, int64_t n, int64_t k, int g, uint8_t* packed, void* scales,
                            void* zeros, hipStream_t st) {
  const int64_t npieces = n * k / 32;
  uint32_t* pk = (uint32_t*)packed;
  TS* sc = (TS*)scales;
  TS* zr = (TS*)zeros;
#ifndef W4_QUANT_PIECES
#define W4_QUANT_PIECES 1
#endif
  constexpr int U = sizeof(TIn) == 2 ? W4_QUANT_PIECES : 1;  // pieces per lane
  const int64_t per_block = 256 * U;
  const dim3 grid((unsigned)((npieces + per_block - 1) / per_block));
  switch (g) {
    case 32:
      k_quantize_pack_sub<TIn, TS, 1, U, SYM><<<grid, 256, 0, st>>>(w, npieces, pk, sc, zr);
      break;
    case 64:
      k_quantize_pack_sub<TIn, TS, 2, U, SYM><<<grid, 256, 0, st>>>(w, npieces, pk, sc, zr);
      break;
    case 128:
      k_quantize_pack_sub<TIn, TS, 4, U, SYM><<<grid, 256, 0, st>>>(w, npieces, pk, sc, zr);
      break;
    case 256:
      k_quantize_pack_sub<TIn, TS, 8, U, SYM><<<grid, 256, 0, st>>>(w, npieces, pk, sc, zr);
      break;
    case 512:
      k_quantize_pack_sub<TIn, TS, 16, U, SYM><<<grid, 256, 0, st>>>(w, npieces, pk, sc, zr);
      break;
    default: {
      const int64_t ngroups = n * (k / g);
      const dim3 g2((unsigned)((ngroups + 3) / 4));
      k_quantize_pack_wave<TIn, TS, SYM><<<g2, 256, 0, st>>>(w, ngroups, g / 8, pk, sc, zr);
    }
  }
  return hipGetLastError();
}

template <bool SYM>
static hipError_t launch_qp_sz(const void* w, int w_dtype, int64_t n, int64_t k, int g,
                               uint8_t* packed, void* scales, void* zeros, int sz_dtype,
                               hipStream_t st) {
  const bool in_bf16 = (w_dtype == W4_BF16);
  const bool s_f16 = (sz_dtype == W4_F16);
  if (in_bf16 && s_f16) return launch_qp<__bf16, _Float16, SYM>(w, n, k, g, packed, scales, zeros, st);
  if (in_bf16) return launch_qp<__bf16, float, SYM>(w, n, k, g, packed, scales, zeros, st);
  if (s_f16) return launch_qp<float, _Float16, SYM>(w, n, k, g, packed, scales, zeros, st);
  return launch_qp<float, float, SYM>(w, n, k, g, packed, scales, zeros, st);
}

hipError_t launch_quantize_pack(const void* w, int w_dtype, int64_t n, int64_t k, int g,
                                uint8_t* packed, void* scales, void* zeros, int sz_dtype,
                                bool symmetric, hipStream_t st) {
  if (symmetric) return launch_qp_sz<true>(w, w_dtype, n, k, g, packed, scales, zeros, sz_dtype, st);
  return launch_qp_sz<false>(w, w_dtype, n, k, g, packed, scales, zeros, sz_dtype, st);
}

// ---------------------------------------------------------------------------
// Calibrated symmetric quantize + pack ("Building a From-Scratch Group-Wise
// INT4 Quantization Layer for LLaMA Weights", Step 4): the group's scale
// comes from a range-clipping calibrator, the codes are the symmetric ones
// above with the stored scale.  One wave per group (g <= 1024); the group's
// values sit in the wave's own LDS region, which needs no barrier (LDS
// operations of a wave complete in order).
//   MODE_PCT: range = the p-th percentile of |w| as torch.quantile computes
//     it in float32: the sorted order statistics i0 = floor(rank) and
//     i1 = ceil(rank), rank = fl32(fl32(p / 100) * (g - 1)), interpolated
//     with f = rank - i0 from the nearer end with one rounding
//     (fma(f, d, a[i0]) for f < 1/2, else fma(f - 1, d, a[i1]), d = a[i1] -
//     a[i0]); the host computes i0, i1 and f.  scale = range / 7.  The order
//     statistics are read from a bitonic sort of |w| in LDS (equal values
//     are equal, so the order of ties does not matter).
//   MODE_MSE: candidate steps from min|w| to max|w| as torch.linspace gives
//     them: d = (hi - lo) / (n - 1), c_i = fma(d, i, lo) for i < n / 2 and
//     fma(-d, n - 1 - i, hi) above; c < 1e-10 is skipped; codes
//     clamp(rint(fl32(w / c)), -7, 7); the error is the float32 sum over the
//     group in column order of (q c - w)^2, divided by g; the first least
//     mean wins (a 64-bit key of the mean's bits and the index; means are
//     non-negative, so their bits order like their values); 1e-8 if no
//     candidate qualifies.  Lane l evaluates candidates l, l + 64, ...
//     The quotient w / c is taken as t = w * r with r = fl32(1 / c), within
//     2^-19 of fl32(w / c) wherever |w / c| <= 8 (r and the product each
//     add at most 2^-24 relative); beyond 8 both clamp to +-7.  A code
//     depends only on which side of a half-integer the quotient falls, so
//     where one of four consecutive t is within 2^-18 of one, the four codes
//     are taken from the correctly rounded division instead.
// ---------------------------------------------------------------------------
constexpr int kCalMaxG = 1024;
enum { MODE_PCT = 0, MODE_MSE = 1 };

__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const uint64_t u = __shfl_xor(v, o, kWave);
    v = u < v ? u : v;
  }
  return v;
}

template <typename TIn, typename TS, int MODE>
__global__ __launch_bounds__(256) void k_quantize_pack_cal(const void* __restrict__ w, int64_t ngroups,
                                                          int cpg, int i0, int i1, float frac, int ncand,
                                                          uint32_t* __restrict__ packed,
                                                          TS* __restrict__ scales,
                                                          TS* __restrict__ zeros) {
  extern __shared__ __attribute__((aligned(16))) float cal_lds[];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t grp = (int64_t)blockIdx.x * 4 + wv;
  if (grp >= ngroups) return;  // uniform per wave; no workgroup barrier follows
  const int g = 8 * cpg;
  int Pg = 32;
  while (Pg < g) Pg <<= 1;
  float* gl = cal_lds + wv * (g + (MODE == MODE_PCT ? Pg : 0));
  const int64_t c0 = grp * cpg;
  for (int c = lane; c < cpg; c += kWave) {
    float v[8];
    Load8<TIn>::run(w, c0 + c, v);
    ((f32x4*)gl)[2 * c] = f32x4{v[0], v[1], v[2], v[3]};
    ((f32x4*)gl)[2 * c + 1] = f32x4{v[4], v[5], v[6], v[7]};
  }
  __builtin_amdgcn_wave_barrier();

  float s32;
  if constexpr (MODE == MODE_PCT) {
    // bitonic sort of |w|, padded with +inf to P = the next power of two,
    // in the LDS region after the group's values; each stage's comparators
    // are spread over the lanes, and a wave's LDS operations complete in
    // order, so stages follow one another with no barrier
    int P = 32;
    while (P < g) P <<= 1;
    float* srt = gl + g;
    for (int e = lane; e < P; e += kWave) srt[e] = e < g ? fabsf(gl[e]) : __builtin_huge_valf();
    for (int k2 = 2; k2 <= P; k2 <<= 1) {
      for (int j = k2 >> 1; j > 0; j >>= 1) {
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        for (int i = lane; i < (P >> 1); i += kWave) {
          const int a = ((i & ~(j - 1)) << 1) | (i & (j - 1));  // comparator i: a, a + j
          const float va = srt[a], vb = srt[a + j];
          const float lo = fminf(va, vb), hi = fmaxf(va, vb);
          const bool up = (a & k2) == 0;
          srt[a] = up ? lo : hi;
          srt[a + j] = up ? hi : lo;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    const float v0 = srt[i0], v1 = srt[i1];
    const float d = v1 - v0;
    const float range = frac < 0.5f ? __builtin_fmaf(frac, d, v0) : __builtin_fmaf(frac - 1.0f, d, v1);
    s32 = range / 7.0f;
  } else {
    float lo = __builtin_huge_valf(), hi = 0.0f;
    for (int e = lane; e < g; e += kWave) {
      const float a = fabsf(gl[e]);
      lo = fminf(lo, a);
      hi = fmaxf(hi, a);
    }
    lo = group_min<kWave>(lo);
    hi = group_max<kWave>(hi);
    const float d = (hi - lo) / (float)(ncand - 1);
    const int half = ncand >> 1;
    auto cand = [&](int i) {
      return i < half ? __builtin_fmaf(d, (float)i, lo) : __builtin_fmaf(-d, (float)(ncand - 1 - i), hi);
    };
    const float gf = (float)g;
    uint64_t best = ~0ull;
    for (int i = lane; i < ncand; i += kWave) {
      const float c = cand(i);
      if (!(c >= 1e-10f)) continue;
      const float r = 1.0f / c;
      float err = 0.0f;
      for (int kk = 0; kk < g; kk += 4) {
        const f32x4 w4 = ((const f32x4*)gl)[kk >> 2];
        float qt[4], dev[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float t = w4[j] * r;
          qt[j] = rintf(t);
          dev[j] = fabsf(t - qt[j]);  // exact; 1/2 at a half-integer
        }
        // any of the four within 2^-18 of a half-integer: the division decides
        if (fmaxf(fmaxf(dev[0], dev[1]), fmaxf(dev[2], dev[3])) > 0.5f - 0x1p-18f) {
#pragma unroll
          for (int j = 0; j < 4; ++j) qt[j] = rintf(w4[j] / c);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float q = __builtin_amdgcn_fmed3f(qt[j], -7.0f, 7.0f);
          const float e = q * c - w4[j];
          err = err + e * e;
        }
      }
      const float mean = err / gf;
      const uint64_t key = ((uint64_t)__float_as_uint(mean) << 32) | (uint32_t)i;
      best = key < best ? key : best;
    }
    best = wave_min_u64(best);
    s32 = best == ~0ull ? 1e-8f : cand((int)(uint32_t)best);
  }
  TS st = (TS)s32;
  if (st == (TS)0.0f) st = (TS)1.0f;
  const float s = (float)st;
  const float r = __builtin_amdgcn_rcpf(s);
  for (int c = lane; c < cpg; c += kWave) {
    const f32x4 a = ((const f32x4*)gl)[2 * c], b = ((const f32x4*)gl)[2 * c + 1];
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    packed[c0 + c] = pack8_sym(v, s, r);
  }
  if (lane == 0) {
    scales[grp] = st;
    zeros[grp] = (TS)8.0f;
  }
}

template <typename TIn, typename TS>
static hipError_t launch_cal_t(const void* w, int64_t n, int64_t k, int g, int mode, double param,
                               uint8_t* packed, void* scales, void* zeros, hipStream_t st) {
  const int64_t ngroups = n * (k / g);
  const dim3 grid((unsigned)((ngroups + 3) / 4));
  int P = 32;
  while (P < g) P <<= 1;
  const size_t lds = (size_t)4 * (g + (mode == MODE_PCT ? P : 0)) * sizeof(float);
  uint32_t* pk = (uint32_t*)packed;
  if (mode == MODE_PCT) {
    // torch.quantile's position of the p-th percentile among g sorted values:
    // the fraction p / 100 as a float32, the rank fraction * (g - 1) in float32
    const float q = (float)(param / 100.0);
    const float rank = q * (float)(g - 1);
    const int i0 = (int)std::floor(rank);
    const int i1 = (int)std::ceil(rank);
    const float f = rank - (float)i0;
    k_quantize_pack_cal<TIn, TS, MODE_PCT><<<grid, 256, lds, st>>>(w, ngroups, g / 8, i0, i1, f, 0, pk,
                                                                     (TS*)scales, (TS*)zeros);
  } else {
    k_quantize_pack_cal<TIn, TS, MODE_MSE><<<grid, 256, lds, st>>>(w, ngroups, g / 8, 0, 0, 0.0f,
                                                                     (int)param, pk, (TS*)scales,
                                                                     (TS*)zeros);
  }
  return hipGetLastError();
}

bool quantize_cal_fits(int g) { return g <= kCalMaxG; }

hipError_t launch_quantize_pack_cal(const void* w, int w_dtype, int64_t n, int64_t k, int g, int mode,
                                    double param, uint8_t* packed, void* scales, void* zeros,
                                    int sz_dtype, hipStream_t st) {
  const bool in_bf16 = (w_dtype == W4_BF16);
  const bool s_f16 = (sz_dtype == W4_F16);
  if (in_bf16 && s_f16) return launch_cal_t<__bf16, _Float16>(w, n, k, g, mode, param, packed, scales, zeros, st);
  if (in_bf16) return launch_cal_t<__bf16, float>(w, n, k, g, mode, param, packed, scales, zeros, st);
  if (s_f16) return launch_cal_t<float, _Float16>(w, n, k, g, mode, param, packed, scales, zeros, st);
  return launch_cal_t<float, float>(w, n, k, g, mode, param, packed, scales, zeros, st);
}

// ---------------------------------------------------------------------------
// Dequantize ("From Scratch: Building a GPTQ INT4 Quantizer in Pure Python",
// Step 4): w = fl32((q - zp) * scale), rounded to the output type.
// One lane per 32-bit word (8 codes); grid-stride over the flat tensor.
// ---------------------------------------------------------------------------
// The group of word c is c >> cpg_log2 when the words per group are a power
// of two (every group size from 32 to 512), else c / cpg.
// fp16 scales: q*s and zp*s are exact in fp32 (4 + 11 significant bits), so
// fma(q, s, -zp*s) rounds the exact (q - zp)*s once, like the definition.
// fp32 scales: the integer q - zp times s, one rounding.
template <typename TS, int OUT, bool POW2>
__global__ __launch_bounds__(256) void k_dequant(const uint32_t* __restrict__ packed,
                                                const void* __restrict__ scales,
                                                const void* __restrict__ zeros, int64_t nchunks,
                                                int cpg, int cpg_log2, void* __restrict__ out) {
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < nchunks;
       c += (int64_t)gridDim.x * 256) {
    const uint32_t word = packed[c];
    const int64_t gi = POW2 ? (c >> cpg_log2) : c / cpg;
    const float s = ScaleT<TS>::load(scales, gi);
    const float zf = ScaleT<TS>::load(zeros, gi);
    float v[8];
    if constexpr (sizeof(TS) == 2) {
      const float b = -zf * s;  // exact
      uint32_t lo = word & 0x0f0f0f0fu, hi = (word >> 4) & 0x0f0f0f0fu;
      // opaque to the optimizer, so each byte converts with v_cvt_f32_ubyteN
      // instead of an extract plus a conversion
      asm("" : "+v"(lo), "+v"(hi));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = fmaf((float)((lo >> (8 * i)) & 0xffu), s, b);
        v[2 * i + 1] = fmaf((float)((hi >> (8 * i)) & 0xffu), s, b);
      }
    } else {
      const int zp = (int)zf;
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (float)((int)((word >> (4 * i)) & 15u) - zp) * s;
    }
    if constexpr (OUT == W4_F32) {
      f32x4* o = (f32x4*)out + 2 * c;
      o[0] = f32x4{v[0], v[1], v[2], v[3]};
      o[1] = f32x4{v[4], v[5], v[6], v[7]};
    } else if constexpr (OUT == W4_BF16) {
      // hardware round-to-nearest-even pairs
      u32x4 r;
      r.x = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)v[0], (__bf16)v[1]});
      r.y = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)v[2], (__bf16)v[3]});
      r.z = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)v[4], (__bf16)v[5]});
      r.w = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)v[6], (__bf16)v[7]});
      ((u32x4*)out)[c] = r;
    } else {
      uint32_t h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = f32_to_f16_bits(v[i]);
      ((u32x4*)out)[c] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                               h[6] | (h[7] << 16)};
    }
  }
}

template <typename TS, bool POW2>
static void launch_dq2(const uint32_t* pk, const void* scales, const void* zeros, int64_t nchunks,
                       int cpg, int lg, void* out, int out_dtype, dim3 grid, hipStream_t st) {
  if (out_dtype == W4_F32)
    k_dequant<TS, W4_F32, POW2><<<grid, 256, 0, st>>>(pk, scales, zeros, nchunks, cpg, lg, out);
  else if (out_dtype == W4_F16)
    k_dequant<TS, W4_F16, POW2><<<grid, 256, 0, st>>>(pk, scales, zeros, nchunks, cpg, lg, out);
  else
    k_dequant<TS, W4_BF16, POW2><<<grid, 256, 0, st>>>(pk, scales, zeros, nchunks, cpg, lg, out);
}

template <typename TS>
static hipError_t launch_dq(const uint8_t* packed, const void* scales, const void* zeros, int64_t n,
                            int64_t k, int g, void* out, int out_dtype, hipStream_t st) {
  const int64_t nchunks = n * k / 8;
  int64_t blocks = (nchunks + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const dim3 grid((unsigned)blocks);
  const uint32_t* pk = (const uint32_t*)packed;
  const int cpg = g / 8;
  if ((cpg & (cpg - 1)) == 0) {
    int lg = 0;
    while ((1 << lg) < cpg) ++lg;
    launch_dq2<TS, true>(pk, scales, zeros, nchunks, cpg, lg, out, out_dtype, grid, st);
  } else {
    launch_dq2<TS, false>(pk, scales, zeros, nchunks, cpg, 0, out, out_dtype, grid, st);
  }
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* packed, const void* scales, const void* zeros,
                          int sz_dtype, int64_t n, int64_t k, int g, void* out, int out_dtype,
                          hipStream_t st) {
  if (sz_dtype == W4_F16)
    return launch_dq<_Float16>(packed, scales, zeros, n, k, g, out, out_dtype, st);
  return launch_dq<float>(packed, scales, zeros, n, k, g, out, out_dtype, st);
}

// ---------------------------------------------------------------------------
// Per-token INT8 activations ("Hands-on Build Guide: Group-wise INT4
// Weight-only Quantization with Per-channel Scales", Step 3).
// One 256-lane block per token: pass 1 finds max|x|, pass 2 (re-reading the
// row from cache) writes clamp(rint(x / s), -128, 127).
// ---------------------------------------------------------------------------
template <typename TX>
__global__ __launch_bounds__(256) void k_act_quant(const void* __restrict__ x, int64_t k,
                                                  int8_t* __restrict__ xq,
                                                  float* __restrict__ x_scale) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int64_t nch = k / 8;
  const int64_t c0 = row * nch;
  float amax = 0.0f;
  for (int64_t c = threadIdx.x; c < nch; c += 256) {
    float v[8];
    Load8<TX>::run(x, c0 + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = group_max<kWave>(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = fmaxf(amax, 1e-8f) / 127.0f;
  for (int64_t c = threadIdx.x; c < nch; c += 256) {
    float v[8];
    Load8<TX>::run(x, c0 + c, v);
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float t = rintf(v[i] / s);
      t = fminf(fmaxf(t, -128.0f), 127.0f);
      b[i] = (uint32_t)((int)t) & 0xffu;
    }
    ((u32x2*)xq)[c0 + c] =
        u32x2{b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
              b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24)};
  }
  if (threadIdx.x == 0) x_scale[row] = s;
}

// Eight activations -> eight int8 codes clamp(rint(x / s), -128, 127), packed
// little-endian.  As in pack8, the division is skipped where it cannot
// change a code: t = x * (1/s) is within 2^-15 of fl32(x / s) because
// |x / s| <= 128 (the hardware reciprocal is within 1 ulp, the product and
// the quotient round once each), and a code only depends on which side of a
// half-integer t lies.  Words with a t within 2^-12 of a half-integer use the
// correctly rounded division.
__device__ __forceinline__ u32x2 act8(const float* v, float s, float r) {
  float c[8];
  float dmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float t = v[i] * r;
    c[i] = rintf(t);
    dmax = fmaxf(dmax, fabsf(t - c[i]));
  }
  if (!(dmax < 0.5f - 0x1p-12f)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = rintf(v[i] / s);
  }
  uint32_t b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = (uint32_t)((int)fminf(fmaxf(c[i], -128.0f), 127.0f)) & 0xffu;
  return u32x2{b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
               b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24)};
}

// Rows of up to 8 NT R activations: one NT-lane block per token, the row held
// in registers (R 8-element chunks per lane) between finding max|x| and
// writing the codes, so it is read once.
template <typename TX, int NT, int R>
__global__ __launch_bounds__(NT) void k_act_quant_reg(const void* __restrict__ x, int64_t k,
                                                     int8_t* __restrict__ xq,
                                                     float* __restrict__ x_scale) {
  __shared__ float red[NT / 64];
  const int64_t row = blockIdx.x;
  const int nch = (int)(k / 8);
  const int64_t c0 = row * nch;
  const int tid = threadIdx.x;
  float v[R][8];
  float amax = 0.0f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = tid + NT * r;
    if (c < nch) {
      Load8<TX>::run(x, c0 + c, v[r]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[r][i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[r][i]));
  }
  amax = group_max<kWave>(amax);
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) amax = fmaxf(amax, red[w]);
  const float s = fmaxf(amax, 1e-8f) / 127.0f;
  const float rs = __builtin_amdgcn_rcpf(s);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = tid + NT * r;
    if (c < nch) ((u32x2*)xq)[c0 + c] = act8(v[r], s, rs);
  }
  if (tid == 0) x_scale[row] = s;
}

hipError_t launch_act_quant(const void* x, int x_dtype, int64_t m, int64_t k, int8_t* xq,
                            float* x_scale, hipStream_t st) {
  const dim3 grid((unsigned)m);
  const bool bf = x_dtype == W4_BF16;
  if (m < 64 && k <= 8 * 1024) {  // few tokens: a wide block per token
    if (bf) k_act_quant_reg<__bf16, 1024, 1><<<grid, 1024, 0, st>>>(x, k, xq, x_scale);
    else k_act_quant_reg<float, 1024, 1><<<grid, 1024, 0, st>>>(x, k, xq, x_scale);
  } else if (k <= 8 * 256 * 4) {
    if (bf) k_act_quant_reg<__bf16, 256, 4><<<grid, 256, 0, st>>>(x, k, xq, x_scale);
    else k_act_quant_reg<float, 256, 4><<<grid, 256, 0, st>>>(x, k, xq, x_scale);
  } else {
    if (bf) k_act_quant<__bf16><<<grid, 256, 0, st>>>(x, k, xq, x_scale);
    else k_act_quant<float><<<grid, 256, 0, st>>>(x, k, xq, x_scale);
  }
  return hipGetLastError();
}

}  // namespace w4
