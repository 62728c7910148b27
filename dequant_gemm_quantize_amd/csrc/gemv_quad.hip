// Small-batch fused dequantize-GEMV for 2 <= M <= 4 bf16 tokens on the
// 4 x 4 x 4 matrix-core shape: v_mfma_f32_4x4x4_16b_bf16 is sixteen
// independent products of a 4 x 4 block of A by a 4 x 4 block of B, one
// block per group of four lanes.  K = 4096, groups a multiple of 32 columns.
//
// Math, per 32-column chunk c of weight row n (inside one group: scale s,
// zero-point zp) and token m:
//   sum_k x[m,k] (q[n,k] - zp) s
//     = s * sum_k x[m,k] (128 + q[n,k])  -  s (128 + zp) * xs[m,c]
// with xs[m,c] the sum of the chunk's activations ("From Scratch: Building a
// GPTQ INT4 Quantizer in Pure Python", Step 4, inside the product of
// "Building a From-Scratch Group-Wise INT4 Quantization Layer for LLaMA
// Weights", Step 2).  128 + q is an exact bfloat16 built from the nibble
// with a shift and one and-or.
//
// Work layout.  Lane l = 4b + q is position q of block b.  In the B operand
// q is a weight row of the current group of four rows, in the A operand q is
// a token, and block b is the 32-column chunk b of a 512-column unit of K.
// So one code load instruction reads 256 contiguous bytes of each of four
// rows, and the eight MFMAs of a 16-byte chunk leave in lane 4b + j the
// chunk's products of row j with all four tokens: the product work does not
// grow with the token count.
//
// A workgroup of W waves owns 4 RQ rows (16); wave w covers units
// [w UPW, (w + 1) UPW) of K for all of them (eight waves of one unit).  The workgroup stages the
// activations once in LDS, already interleaved into the codes' pair order,
// with their chunk sums, and the scale / zero-point tile as (s, -s(128+zp))
// pairs, while the codes are in flight; each wave then reads its units'
// activations into registers.  At the end each wave sums its 16 blocks with
// a transposing butterfly and the waves' sums meet in LDS.
#include "w4_common.h"
#include "w4_internal.h"

namespace w4 {

namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Eight waves of one unit each: on [11008,4096] at 2 / 3 / 4 tokens
// 7.8 / 7.9 / 8.3 us against 7.7-8.0 / 8.5 / 8.7-8.8 us with four waves of
// two units (same box, alternating runs), and faster on [4096,4096] at every
// token count; 32 rows per workgroup were slower with either.
#ifndef W4_QUAD_WAVES
#define W4_QUAD_WAVES 8
#endif
constexpr int kQW = W4_QUAD_WAVES;  // waves per workgroup
#ifndef W4_QUAD_RQ
#define W4_QUAD_RQ 4
#endif
constexpr int kQRQ = W4_QUAD_RQ;    // groups of four rows per workgroup
constexpr int kQUPW = 8 / kQW;      // 512-column units per wave
constexpr int kQK = 512 * kQW * kQUPW;  // K
constexpr int kQRows = 4 * kQRQ;
constexpr int kQThr = 64 * kQW;

template <typename TS> struct QSZ;
template <> struct QSZ<_Float16> {
  typedef uint16_t T;
  __device__ static float f(T v) { return (float)__builtin_bit_cast(_Float16, v); }
};
template <> struct QSZ<float> {
  typedef uint32_t T;
  __device__ static float f(T v) { return __uint_as_float(v); }
};

template <typename TY>
__device__ __forceinline__ void put_y(void* y, int64_t i, float v) {
  if constexpr (sizeof(TY) == 4) {
    ((float*)y)[i] = v;
  } else {
    ((uint16_t*)y)[i] = (uint16_t)f32_to_bf16_bits(v);
  }
}

__device__ __forceinline__ bf16x4 pair2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(bf16x4, u32x2{a, b});
}

// s + the two bf16 of a pair.  The pair is taken by value: a bit cast of a
// vector element in place reads the vector's first element whatever the
// element named.
__device__ __forceinline__ float add_pair(uint32_t a, float s) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, 0x3f803f80u),
                                         s, false);
}

template <int CTRL>
__device__ __forceinline__ float qdpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf,
                                                               false));
}

// One exchange across lane bit MASK of the values a lane still holds: with
// the bit set a lane keeps the upper half of its list, else the lower half,
// and adds the partner's copy of the same half.
template <int NV, int MASK>
__device__ __forceinline__ void halve(float (&v)[NV], int lane) {
  constexpr int half = NV / 2;
  const bool hi = lane & MASK;
#pragma unroll
  for (int k = 0; k < half; ++k) {
    const float keep = hi ? v[half + k] : v[k];
    const float send = hi ? v[k] : v[half + k];
    v[k] = keep + __shfl_xor(send, MASK, kWave);
  }
}

// Sum over the 16 lanes of equal lane mod 4 (lane bits 2..5) of NV values
// per lane (NV = 4, 8, 16 or 32): exchanges over bits 5, 4, ... while more
// than one value is left, then plain sums over the remaining bits.  For
// NV <= 16 lane 4b + j ends with the full sum of value b >> (4 - log2 NV) in
// v[0]; for NV = 32 with the sums of values 2b and 2b + 1 in v[0], v[1].
template <int NV>
__device__ __forceinline__ void sum_blocks(float (&v)[NV], int lane) {
  static_assert(NV == 4 || NV == 8 || NV == 16 || NV == 32, "4, 8, 16 or 32 values");
  halve<NV, 32>(v, lane);
  halve<NV / 2, 16>(*reinterpret_cast<float(*)[NV / 2]>(&v), lane);
  if constexpr (NV >= 8) {
    halve<NV / 4, 8>(*reinterpret_cast<float(*)[NV / 4]>(&v), lane);
  } else {
    v[0] += __shfl_xor(v[0], 8, kWave);
  }
  if constexpr (NV >= 16) {
    halve<NV / 8, 4>(*reinterpret_cast<float(*)[NV / 8]>(&v), lane);
  } else {
    v[0] += __shfl_xor(v[0], 4, kWave);
  }
}

}  // namespace

// MT: tokens (2..4; M == MT).  cpg = g / 32 chunks per group; gmagic =
// ceil(2^32 / cpg), or 0 when cpg == 1 (group = chunk): umulhi(c, gmagic) ==
// c / cpg for every chunk index c < 128.
// LDS: x_l [MT][K/8] 16-byte groups; xs_l [K/32][4] chunk sums (token
// minor); sz_l [RW][ng] (s, -s (128 + zp)); red_l [W][64] wave sums.
template <typename TS, typename TY, int MT>
__global__ __launch_bounds__(kQThr) void k_w4a16_quad(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ packed,
    const void* __restrict__ scales, const void* __restrict__ zeros, int64_t N, int ng,
    uint32_t gmagic, void* __restrict__ y) {
  constexpr int K = kQK, RQ = kQRQ, UPW = kQUPW, W = kQW;
  constexpr int NV = 4 * RQ * (MT <= 1 ? 1 : MT <= 2 ? 2 : 4) / 4;  // partial sums kept per lane
  constexpr int TI = NV / RQ;                                           // token slots per row group
  typedef typename QSZ<TS>::T R;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  u32x4* x_l = (u32x4*)lds;                                         // [MT][K/8]
  float* xs_l = (float*)(lds + MT * (K / 8) * 16);                  // [K/32][4]
  float2* sz_l = (float2*)(lds + MT * (K / 8) * 16 + (K / 32) * 16);  // [RW][ng]
  float* red_l = (float*)(sz_l + kQRows * ng);                      // [W][64]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane & 3;
  const int b = lane >> 2;
  const int64_t n0 = (int64_t)blockIdx.x * kQRows;
  const int u0 = wave * UPW;

  // ---- 1. staging loads: activations, then the scale / zero-point tile ----
  constexpr int XPER = MT * (K / 8) / kQThr;  // exact: 16-byte groups per thread
  u32x4 xv[XPER];
#pragma unroll
  for (int r = 0; r < XPER; ++r) xv[r] = *(const u32x4*)((const char*)x + (uint32_t)(tid + kQThr * r) * 16u);
  const int64_t nvalid = N - n0 < kQRows ? N - n0 : kQRows;
  const int tvalid = (int)nvalid * ng;
  const int tsize = kQRows * ng;
  constexpr int SMAX = 8;
  const int sper = (tsize + kQThr - 1) / kQThr;  // <= SMAX (checked on the host)
  const char* sbase = (const char*)scales + n0 * ng * (int64_t)sizeof(R);
  const char* zbase = (const char*)zeros + n0 * ng * (int64_t)sizeof(R);
  R sv[SMAX], zv[SMAX];
#pragma unroll
  for (int r = 0; r < SMAX; ++r) {
    if (r < sper) {
      const int e = tid + kQThr * r;
      const uint32_t off = (uint32_t)(e < tvalid ? e : tvalid - 1) * (uint32_t)sizeof(R);
      sv[r] = *(const R*)(sbase + off);
      zv[r] = *(const R*)(zbase + off);
    }
  }

  // ---- 2. codes: RQ x UPW 16-byte loads per lane ---------------------------
  // lane (q, b), row group r, unit u: row n0 + 4 r + q, chunk 16 (u0 + u) + b
  const __amdgpu_buffer_rsrc_t wrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(packed + n0 * (K / 2)), (short)0, 0x7fffffff,
                                        0x00020000);
  u32x4 cw[RQ][UPW];
#pragma unroll
  for (int r = 0; r < RQ; ++r) {
    const int64_t row = n0 + 4 * r + q < N ? n0 + 4 * r + q : N - 1;
    const uint32_t vo = (uint32_t)((row - n0) * (K / 2)) + (uint32_t)(u0 * 256 + b * 16);
#pragma unroll
    for (int u = 0; u < UPW; ++u)
      cw[r][u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, vo, u * 256, 2));
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- 3. LDS: interleaved activations with chunk sums, the tile ----------
  // the four 16-byte groups of a chunk sit in threads 4j .. 4j+3 (K/8 is a
  // multiple of 4): two row shifts gather the chunk sum in thread 4j + 3
#pragma unroll
  for (int r = 0; r < XPER; ++r) {
    const u32x4 a = xv[r];
    u32x4 o;
    o.x = __builtin_amdgcn_perm(a.z, a.x, 0x05040100u);
    o.y = __builtin_amdgcn_perm(a.z, a.x, 0x07060302u);
    o.z = __builtin_amdgcn_perm(a.w, a.y, 0x05040100u);
    o.w = __builtin_amdgcn_perm(a.w, a.y, 0x07060302u);
    const int i = tid + kQThr * r;
    x_l[i] = o;
    float p = add_pair(a.x, 0.0f);
    p = add_pair(a.y, p);
    p = add_pair(a.z, p);
    p = add_pair(a.w, p);
    p += qdpp<0x111>(p);  // row_shr:1
    p += qdpp<0x112>(p);  // row_shr:2
    const int m = i / (K / 8), c = (i % (K / 8)) >> 2;
    if ((tid & 3) == 3) xs_l[c * 4 + m] = p;
  }
#pragma unroll
  for (int r = 0; r < SMAX; ++r) {
    if (r < sper) {
      const int e = tid + kQThr * r;
      if (e < tsize) {
        const float s = QSZ<TS>::f(sv[r]);
        sz_l[e] = make_float2(s, -s * (128.0f + QSZ<TS>::f(zv[r])));
      }
    }
  }
  int grp[UPW];
#pragma unroll
  for (int u = 0; u < UPW; ++u) {
    const uint32_t c = (uint32_t)(16 * (u0 + u) + b);
    grp[u] = gmagic ? (int)__umulhi(c, gmagic) : (int)c;
  }
  __syncthreads();

  // ---- 4. the wave's activations (token min(q, MT - 1)) and chunk sums ----
  const int tq = q < MT ? q : MT - 1;
  uint32_t xi[UPW][16];
  float xq[UPW][4];
#pragma unroll
  for (int u = 0; u < UPW; ++u) {
    const int c = 16 * (u0 + u) + b;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const u32x4 a = x_l[tq * (K / 8) + 4 * c + v];
      xi[u][4 * v + 0] = a.x;
      xi[u][4 * v + 1] = a.y;
      xi[u][4 * v + 2] = a.z;
      xi[u][4 * v + 3] = a.w;
    }
    const f32x4 s4 = *(const f32x4*)(xs_l + 4 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) xq[u][i] = i < MT ? s4[i] : 0.0f;
  }

  // ---- 5. products, in the order the codes were loaded ---------------------
  const NibConst nk = NibConst::make();
  float acc[RQ][TI];
#pragma unroll
  for (int r = 0; r < RQ; ++r)
#pragma unroll
    for (int i = 0; i < TI; ++i) acc[r][i] = 0.0f;
#pragma unroll
  for (int r = 0; r < RQ; ++r) {
#pragma unroll
    for (int u = 0; u < UPW; ++u) {
      const float2 sz = sz_l[(4 * r + q) * ng + grp[u]];
      const uint32_t w4[4] = {cw[r][u].x, cw[r][u].y, cw[r][u].z, cw[r][u].w};
      f32x4 ga = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint32_t c0 = nk(w4[v]), c1 = nk(w4[v] >> 4), c2 = nk(w4[v] >> 8), c3 = nk(w4[v] >> 12);
        ga = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(pair2(xi[u][4 * v], xi[u][4 * v + 1]), pair2(c0, c1), ga,
                                                    0, 0, 0);
        ga = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(pair2(xi[u][4 * v + 2], xi[u][4 * v + 3]), pair2(c2, c3),
                                                    ga, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < TI; ++i) acc[r][i] = fmaf(sz.x, ga[i], fmaf(sz.y, xq[u][i], acc[r][i]));
    }
  }

  // ---- 6. sum over the 16 blocks, then over the waves ----------------------
  // value index k = TI r + i: token i of row 4 r + j
  float v[NV];
#pragma unroll
  for (int r = 0; r < RQ; ++r)
#pragma unroll
    for (int i = 0; i < TI; ++i) v[TI * r + i] = acc[r][i];
  sum_blocks<NV>(v, lane);
  constexpr int P = NV > 16 ? NV / 16 : 1;  // sums per lane
#pragma unroll
  for (int p = 0; p < P; ++p) red_l[(wave * 64 + lane) * P + p] = v[p];
  __syncthreads();
  if (wave == 0) {
    constexpr int SH = NV >= 16 ? 0 : NV == 8 ? 1 : 2;  // lanes holding copies of one sum
#pragma unroll
    for (int p = 0; p < P; ++p) {
      float s = red_l[lane * P + p];
#pragma unroll
      for (int w = 1; w < W; ++w) s += red_l[(w * 64 + lane) * P + p];
      const int k = (b >> SH) * P + p;
      const int i = k % TI, r = k / TI;
      const int64_t n = n0 + 4 * r + q;
      if ((b & ((1 << SH) - 1)) == 0 && i < MT && n < N) put_y<TY>(y, (int64_t)i * N + n, s);
    }
  }
}

size_t quad_lds_bytes(int64_t m, int64_t k, int g) {
  return (size_t)(m * (k / 8) * 16 + (k / 32) * 16 + kQRows * (k / g) * 8 + kQW * 64 * 4 * (kQRQ > 4 ? 2 : 1));
}

// Shapes the kernel takes: 2 <= M <= 4, K = 4096, g a multiple of 32
// dividing K with a scale tile of at most eight elements per thread.
bool quad_fits(int64_t m, int64_t k, int g) {
  if (m < 2 || m > 4 || k != kQK || g <= 0 || g % 32 != 0 || k % g != 0) return false;
  return (kQRows * (k / g) + kQThr - 1) / kQThr <= 8;
}

template <typename TS, typename TY>
static void quad_go(int M, dim3 grid, size_t lds, hipStream_t st, const uint16_t* x, const uint8_t* packed,
                    const void* scales, const void* zeros, int64_t n, int ng, uint32_t gmagic, void* y) {
  if (M == 2) k_w4a16_quad<TS, TY, 2><<<grid, kQThr, lds, st>>>(x, packed, scales, zeros, n, ng, gmagic, y);
  else if (M == 3) k_w4a16_quad<TS, TY, 3><<<grid, kQThr, lds, st>>>(x, packed, scales, zeros, n, ng, gmagic, y);
  else k_w4a16_quad<TS, TY, 4><<<grid, kQThr, lds, st>>>(x, packed, scales, zeros, n, ng, gmagic, y);
}

hipError_t launch_w4a16_quad(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                             const void* scales, const void* zeros, int sz_dtype, int64_t n,
                             int g, void* y, int y_dtype, hipStream_t st) {
  if (!quad_fits(m, k, g)) return hipErrorInvalidValue;
  const int ng = (int)(k / g);
  const int cpg = g / 32;
  const uint32_t gmagic = cpg == 1 ? 0u : (uint32_t)((0x100000000ull + cpg - 1) / cpg);
  const size_t lds = quad_lds_bytes(m, k, g);
  const dim3 grid((unsigned)((n + kQRows - 1) / kQRows));
  const uint16_t* xb = (const uint16_t*)x;
  const int M = (int)m;
  if (sz_dtype == W4_F16) {
    if (y_dtype == W4_F32) quad_go<_Float16, float>(M, grid, lds, st, xb, packed, scales, zeros, n, ng, gmagic, y);
    else quad_go<_Float16, __bf16>(M, grid, lds, st, xb, packed, scales, zeros, n, ng, gmagic, y);
  } else {
    if (y_dtype == W4_F32) quad_go<float, float>(M, grid, lds, st, xb, packed, scales, zeros, n, ng, gmagic, y);
    else quad_go<float, __bf16>(M, grid, lds, st, xb, packed, scales, zeros, n, ng, gmagic, y);
  }
  return hipGetLastError();
}

}  // namespace w4
