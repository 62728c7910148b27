// Decode fused dequantize-GEMV for one bf16 token (the kernel is written for
// MT tokens; only MT = 1 is launched), group sizes of at least 128 columns.
// VALU-only: no MFMA.
//
// Math, per 32-column chunk c of weight row n (inside one group: scale s,
// zero-point zp) and token m:
//   sum_k x[m,k] (q[n,k] - zp) s
//     = s * sum_k x[m,k] (128 + q[n,k])  -  s (128 + zp) * xs[m,c]
// with xs[m,c] = sum of the chunk's activations ("From Scratch: Building a
// GPTQ INT4 Quantizer in Pure Python", Step 4, inside the product of
// "Building a From-Scratch Group-Wise INT4 Quantization Layer for LLaMA
// Weights", Step 2).  128 + q is an exact bfloat16 built from the nibble
// with a shift and one and-or; v_dot2_f32_bf16 multiplies two such codes by
// two activations and accumulates in fp32.
//
// Work layout.  A workgroup of W waves owns W * RW weight rows; wave w owns
// rows RW*w .. RW*w + RW-1 over all of K.  Lane l covers the 16-byte chunks l, l+64, ...
// of a row (32 columns each), so every load instruction reads 1 KB of one
// row contiguously.  The workgroup stages the activations in LDS once,
// already interleaved into the codes' pair order, with their chunk sums xs;
// each lane reads its columns into registers and reuses them for the wave's
// rows.  The rows' 64 partial sums are added together at the end (quad
// exchanges, DPP row shifts, two cross-row shuffles).
#include "w4_common.h"
#include "w4_internal.h"

namespace w4 {

namespace {

#ifndef W4_DOT2_RW
#define W4_DOT2_RW 4
#endif
#ifndef W4_DOT2_WAVES
#define W4_DOT2_WAVES 4
#endif
constexpr int kWavesWg = W4_DOT2_WAVES;         // waves per workgroup
constexpr int kThreads = 64 * kWavesWg;
// Weight rows per wave: W4_DOT2_RW up to K = 8192; two above, where the
// codes and activations of six chunk rounds leave registers for no more
// (measured on [4096,11008]: 9.0 us with two rows, 10.0 with four).
constexpr int rows_wave(int ch) { return ch <= 4 ? W4_DOT2_RW : 2; }

// 8 codes of a word -> 4 bf16 pairs (128 + q) in the order (0,4),(1,5),(2,6),(3,7).
__device__ __forceinline__ void codes8(uint32_t p, const NibConst& nk, uint32_t (&o)[4]) {
  o[0] = nk(p);
  o[1] = nk(p >> 4);
  o[2] = nk(p >> 8);
  o[3] = nk(p >> 12);
}

// 8 bf16 activations (4 pairs, natural order) -> pairs (x0,x4),(x1,x5),(x2,x6),(x3,x7).
__device__ __forceinline__ void interleave(const u32x4 v, uint32_t (&o)[4]) {
  o[0] = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
  o[1] = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
  o[2] = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
  o[3] = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf,
                                                               0xf, false));
}

// Sums over the 64 lanes of R per-lane values a[0..R-1] (R = 2 or 4) at
// once: two quad exchanges leave lane l with the 4-lane partial of value
// l mod R (l mod 4 for R = 4, each class held twice per quad for R = 2), row
// shifts finish the rows of 16 lanes, and two cross-row shuffles the wave.
// Lane 64 - R + j returns the total of a[j].
template <int R>
__device__ __forceinline__ float wave_sum_rows(const float (&a)[R], int lane) {
  static_assert(R == 2 || R == 4, "two or four values");
  constexpr int kXor1 = 0xB1, kXor2 = 0x4E;  // quad_perm [1,0,3,2], [2,3,0,1]
  const bool odd = lane & 1;
  float v;
  if constexpr (R == 4) {
    const float v01 = (odd ? a[1] : a[0]) + dpp<kXor1>(odd ? a[0] : a[1]);
    const float v23 = (odd ? a[3] : a[2]) + dpp<kXor1>(odd ? a[2] : a[3]);
    const bool hi = lane & 2;
    v = (hi ? v23 : v01) + dpp<kXor2>(hi ? v01 : v23);
  } else {
    v = (odd ? a[1] : a[0]) + dpp<kXor1>(odd ? a[0] : a[1]);
    v += dpp<kXor2>(v);
  }
  v += dpp<0x114>(v);  // row_shr:4 (lanes shifted in from outside the row add 0)
  v += dpp<0x118>(v);  // row_shr:8
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

template <typename TY>
__device__ __forceinline__ void put(void* y, int64_t i, float v) {
  if constexpr (sizeof(TY) == 4) {
    ((float*)y)[i] = v;
  } else {
    ((uint16_t*)y)[i] = (uint16_t)f32_to_bf16_bits(v);
  }
}

// Raw scale / zero-point element (loaded unconverted, converted later).
template <typename TS> struct SZ;
template <> struct SZ<_Float16> {
  typedef uint16_t T;
  __device__ static float f(T v) { return (float)__builtin_bit_cast(_Float16, v); }
};
template <> struct SZ<float> {
  typedef uint32_t T;
  __device__ static float f(T v) { return __uint_as_float(v); }
};

}  // namespace

// CH: 16-byte chunks (32 columns) per lane and row, K <= 2048 CH.  Lane l
// takes chunks l, l + 64, ...; chunks past the row's K / 32 reuse its last
// chunk's addresses and contribute nothing (zero scale pair).  FULL: K is
// exactly 2048 CH, so no chunk lies past the row and no index needs a clamp.
// ng = K / g groups per row; cpg_magic = ceil(2^32 / cpg) for cpg = g / 32
// chunks per group, so that umulhi(ci, cpg_magic) == ci / cpg exactly for
// every chunk index (ci * cpg^2 < 2^32 holds for ci < 384, cpg <= 384).
template <typename TS, typename TY, int MT, int CH, bool FULL>
__global__ __launch_bounds__(kThreads) void k_w4a16_dot2(
    const uint16_t* __restrict__ x, int M, int K, const uint8_t* __restrict__ packed,
    const void* __restrict__ scales, const void* __restrict__ zeros, int64_t N, int ng,
    uint32_t cpg_magic, void* __restrict__ y) {
  // LDS: activations [MT][K] bf16, each 16-byte group interleaved into the
  // codes' pair order; their 32-column chunk sums [MT][K/32]; scale tile
  // [rows][ng] as (s, -s*(128+zp)) float pairs.  Each region is rounded up
  // to the staging lanes.
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  constexpr int kRowsWave = rows_wave(CH);
  constexpr int kRowsWg = kWavesWg * kRowsWave;
  constexpr int XPER_ = (MT * CH * 2048 / 8 + kThreads - 1) / kThreads;
  u32x4* x_l = (u32x4*)lds;
  float* xsum_l = (float*)(lds + XPER_ * kThreads * 16);
  float2* sz_l = (float2*)(lds + XPER_ * kThreads * 20);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t n0 = (int64_t)blockIdx.x * kRowsWg;

  // ---- 1. staging loads (activations, scale / zero-point tile), straight
  //         line: XPER / SPER per thread, indices clamped into range.  All
  //         addresses are a uniform base plus a 32-bit lane offset. --------
  constexpr int XPER = XPER_;  // 16-byte activation groups per thread
  // FULL: XPER * kThreads == MT * K / 8 exactly
  const int xgroups = MT * (K / 8);
  const char* xg = (const char*)x;
  u32x4 xv[XPER];
#pragma unroll
  for (int r = 0; r < XPER; ++r) {
    int i = tid + kThreads * r;
    if constexpr (!FULL) i = i < xgroups ? i : xgroups - 1;
    xv[r] = *(const u32x4*)(xg + (uint32_t)i * 16u);
  }
  // The workgroup's rows are consecutive, so their scales (and zeros) are
  // one contiguous run of rows * ng elements; rows past N are never stored,
  // so their slots just repeat the last valid element.
  constexpr int SPER = (kRowsWg * 16 * CH + kThreads - 1) / kThreads;  // >= kRowsWg * ng
  typedef typename SZ<TS>::T R;
  const int64_t nrows_valid = N - n0 < kRowsWg ? N - n0 : kRowsWg;
  const int tvalid = (int)nrows_valid * ng;
  const char* sbase = (const char*)scales + n0 * ng * (int64_t)sizeof(R);
  const char* zbase = (const char*)zeros + n0 * ng * (int64_t)sizeof(R);
  R sv[SPER], zv[SPER];
#pragma unroll
  for (int r = 0; r < SPER; ++r) {
    const int e = tid + kThreads * r;
    const uint32_t off = (uint32_t)(e < tvalid ? e : tvalid - 1) * (uint32_t)sizeof(R);
    sv[r] = *(const R*)(sbase + off);
    zv[r] = *(const R*)(zbase + off);
  }

  // ---- 2. codes of the wave's rows: kRowsWave x CH 16-byte loads per lane --
  const int nchunk = K / 32;
  u32x4 wq[kRowsWave][CH];
#pragma unroll
  for (int r = 0; r < kRowsWave; ++r) {
    int64_t n = n0 + wave * kRowsWave + r;
    n = n < N ? n : N - 1;
    const char* row = (const char*)packed + n * (int64_t)(K / 2);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      int ci = lane + 64 * c;
      if constexpr (!FULL) ci = ci < nchunk ? ci : nchunk - 1;
      wq[r][c] = __builtin_nontemporal_load((const u32x4*)(row + (uint32_t)ci * 16u));
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- 3. LDS stores (wait for the staging loads only) ---------------------
  // unconditional: the LDS regions have room for every staging lane.  The
  // four 16-byte groups of a 32-column chunk sit in lanes 4j .. 4j+3, so two
  // row shifts gather the chunk's sum in lane 4j+3.
#pragma unroll
  for (int r = 0; r < XPER; ++r) {
    uint32_t o[4];
    interleave(xv[r], o);
    x_l[tid + kThreads * r] = u32x4{o[0], o[1], o[2], o[3]};
    float p = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t) p = dot2(o[t], 0x3f803f80u, p);  // + x_a * 1.0 + x_b * 1.0
    p += dpp<0x111>(p);  // row_shr:1
    p += dpp<0x112>(p);  // row_shr:2
    if ((tid & 3) == 3) xsum_l[(tid + kThreads * r) >> 2] = p;
  }
#pragma unroll
  for (int r = 0; r < SPER; ++r) {
    const float sf = SZ<TS>::f(sv[r]);
    sz_l[tid + kThreads * r] = float2{sf, -sf * (128.0f + SZ<TS>::f(zv[r]))};
  }
  __syncthreads();

  // ---- activations of this lane's columns (interleaved) and chunk sums ----
  uint32_t xa[MT][CH][16];
  float xs[MT][CH];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      // columns 32*(lane + 64c) .. +31 = 16-byte groups 4*(lane + 64c) .. +3
      // (past K: the staged copies of the last group, never used)
      int ci = lane + 64 * c;
      if constexpr (!FULL) ci = ci < nchunk ? ci : nchunk - 1;
      const u32x4* src = x_l + m * (K / 8) + 4 * ci;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 v = src[q];
        xa[m][c][4 * q + 0] = v.x;
        xa[m][c][4 * q + 1] = v.y;
        xa[m][c][4 * q + 2] = v.z;
        xa[m][c][4 * q + 3] = v.w;
      }
      xs[m][c] = xsum_l[m * (K / 32) + ci];
    }

  // ---- rows: dot products, scale, zero-point correction, wave sums --------
  const NibConst nk = NibConst::make();
  int gq[CH];  // group of the lane's chunk c, or -1 past the row's end
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ci = lane + 64 * c;
    gq[c] = (int)__umulhi((uint32_t)ci, cpg_magic);
    if constexpr (!FULL) gq[c] = ci < nchunk ? gq[c] : -1;
  }
  float acc[MT][kRowsWave];
#pragma unroll
  for (int r = 0; r < kRowsWave; ++r) {
    const int rr = wave * kRowsWave + r;
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m][r] = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      float2 sc = sz_l[rr * ng + (gq[c] >= 0 ? gq[c] : 0)];
      if constexpr (!FULL) sc = gq[c] >= 0 ? sc : float2{0.0f, 0.0f};
      const uint32_t w4[4] = {wq[r][c].x, wq[r][c].y, wq[r][c].z, wq[r][c].w};
      float d[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) d[m] = 0.0f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uint32_t b[4];
        codes8(w4[t], nk, b);
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int u = 0; u < 4; ++u) d[m] = dot2(b[u], xa[m][c][4 * t + u], d[m]);
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m][r] = fmaf(sc.x, d[m], fmaf(sc.y, xs[m][c], acc[m][r]));
    }
  }
  // ---- wave sums of the rows; lane 64 - kRowsWave + j stores row j --------
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const float tot = wave_sum_rows<kRowsWave>(acc[m], lane);
    const int64_t n = n0 + wave * kRowsWave + (lane & (kRowsWave - 1));
    if (lane >= 64 - kRowsWave && m < M && n < N) put<TY>(y, (int64_t)m * N + n, tot);
  }
}

static int dot2_ch(int64_t k) { return (int)((k + 2047) / 2048); }

size_t dot2_lds_bytes(int64_t m, int64_t k, int g) {
  (void)g;
  const int ch = dot2_ch(k);
  const int rows_wg = kWavesWg * rows_wave(ch);
  const int64_t xper = (m * ch * 2048 / 8 + kThreads - 1) / kThreads;
  return (size_t)(xper * kThreads * 20 + ((rows_wg * 16 * ch + kThreads - 1) / kThreads) * kThreads * 8);
}

bool dot2_fits(int64_t m, int64_t k, int g) {
  // One token: two already run faster in the LDS decode kernel (8.3 against
  // 9.5 us on [11008,4096]).  Groups of at least 128 keep the scale tile
  // within 16 CH pairs per row.
  return m == 1 && g >= 128 && k % 32 == 0 && k <= 6 * 2048;
}

template <typename TS, typename TY, int MT, bool FULL>
static void dot2_go(dim3 grid, hipStream_t st, const uint16_t* x, int64_t k, const uint8_t* packed,
                    const void* scales, const void* zeros, int64_t n, int g, void* y) {
  const size_t lds = dot2_lds_bytes(MT, k, g);
  const uint32_t cpg = (uint32_t)(g / 32);
  const uint32_t magic = (uint32_t)((((uint64_t)1 << 32) + cpg - 1) / cpg);
  const int ki = (int)k, ng = (int)(k / g);
#define W4_DOT2_CASE(C)                                                                          \
  k_w4a16_dot2<TS, TY, MT, C, FULL><<<grid, kThreads, lds, st>>>(x, MT, ki, packed, scales, zeros, \
                                                                 n, ng, magic, y)
  switch (dot2_ch(k)) {
    case 1: W4_DOT2_CASE(1); break;
    case 2: W4_DOT2_CASE(2); break;
    case 3: W4_DOT2_CASE(3); break;
    case 4: W4_DOT2_CASE(4); break;
    case 5: W4_DOT2_CASE(5); break;
    default: W4_DOT2_CASE(6); break;
  }
#undef W4_DOT2_CASE
}

template <typename TS, typename TY>
static void dot2_full(dim3 grid, hipStream_t st, const uint16_t* x, int64_t k, const uint8_t* packed,
                      const void* scales, const void* zeros, int64_t n, int g, void* y) {
  if (k % 2048 == 0) dot2_go<TS, TY, 1, true>(grid, st, x, k, packed, scales, zeros, n, g, y);
  else dot2_go<TS, TY, 1, false>(grid, st, x, k, packed, scales, zeros, n, g, y);
}

hipError_t launch_w4a16_dot2(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                             const void* scales, const void* zeros, int sz_dtype, int64_t n,
                             int g, void* y, int y_dtype, hipStream_t st) {
  const int rows_wg = kWavesWg * rows_wave(dot2_ch(k));
  const dim3 grid((unsigned)((n + rows_wg - 1) / rows_wg));
  const uint16_t* xb = (const uint16_t*)x;
  const bool sh = sz_dtype == W4_F16, yf = y_dtype == W4_F32;
  (void)m;  // one token (dot2_fits)
  if (sh && yf) dot2_full<_Float16, float>(grid, st, xb, k, packed, scales, zeros, n, g, y);
  else if (sh) dot2_full<_Float16, __bf16>(grid, st, xb, k, packed, scales, zeros, n, g, y);
  else if (yf) dot2_full<float, float>(grid, st, xb, k, packed, scales, zeros, n, g, y);
  else dot2_full<float, __bf16>(grid, st, xb, k, packed, scales, zeros, n, g, y);
  return hipGetLastError();
}

}  // namespace w4
