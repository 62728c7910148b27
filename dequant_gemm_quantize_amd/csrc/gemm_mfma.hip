// Prefill fused dequantize-GEMM: y = x . dequant(W)^T for many tokens (bf16
// x), bf16 MFMA with fp32 accumulation.  MFMA-bound at M = 2048.
//
// Math ("Building a From-Scratch Group-Wise INT4 Quantization Layer for
// LLaMA Weights", Step 2, with the dequantization of "From Scratch: Building
// a GPTQ INT4 Quantizer in Pure Python", Step 4): every weight tile is
// dequantized once per workgroup to bf16, w = RNE((q - zp) * s) -- computed
// as fma(q, s, -zp*s), exact in fp32 before the one rounding -- and written
// to LDS, where it feeds v_mfma_f32_32x32x16_bf16 together with the
// activation tile.  No dequantized matrix ever reaches memory.
//
// Tiling.  Workgroup tile 256 (M) x 128 (N), K in steps of 64, both operand
// tiles double-buffered in LDS (rows padded by 16 bytes).  Four waves in a
// 2 x 2 arrangement, each owning a 128 x 64 block of the output: 4 x 2 MFMA
// tiles of 32 x 32, 128 fp32 accumulators per lane.  The next K step's
// global loads are in flight while the current one runs on the MFMA units.
// Tiles are numbered so that consecutive workgroups (which the dispatcher
// spreads over the 8 XCDs) share an N block and each XCD keeps working on
// the same M block of x, which then stays in that XCD's L2.
#include "w4_common.h"
#include "w4_internal.h"

namespace w4 {

namespace {

constexpr int BM = 256, BN = 128, BK = 64;
constexpr int LDS_ROW = BK + 8;  // bf16 elements per LDS row (+16 bytes of padding)
constexpr int A_STAGE = BM * LDS_ROW;
constexpr int B_STAGE = BN * LDS_ROW;
constexpr size_t kGemmLds = (size_t)2 * (A_STAGE + B_STAGE) * 2;

template <typename TS> struct GS;
template <> struct GS<_Float16> {
  typedef uint16_t T;
  __device__ static float f(T v) { return (float)__builtin_bit_cast(_Float16, v); }
};
template <> struct GS<float> {
  typedef uint32_t T;
  __device__ static float f(T v) { return __uint_as_float(v); }
};

// 8 codes of a packed word -> 8 bf16 weights (natural column order),
// w = RNE(fma(q, s, b)) with b = -zp * s.
__device__ __forceinline__ u32x4 dequant8(uint32_t p, float s, float b) {
  const uint32_t lo = p & 0x0f0f0f0fu;         // codes 0, 2, 4, 6
  const uint32_t hi = (p >> 4) & 0x0f0f0f0fu;  // codes 1, 3, 5, 7
  float w[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w[2 * i] = fmaf((float)((lo >> (8 * i)) & 0xffu), s, b);
    w[2 * i + 1] = fmaf((float)((hi >> (8 * i)) & 0xffu), s, b);
  }
  u32x4 r;
  bf16x2 t;
  t = bf16x2{(__bf16)w[0], (__bf16)w[1]}; r.x = __builtin_bit_cast(uint32_t, t);
  t = bf16x2{(__bf16)w[2], (__bf16)w[3]}; r.y = __builtin_bit_cast(uint32_t, t);
  t = bf16x2{(__bf16)w[4], (__bf16)w[5]}; r.z = __builtin_bit_cast(uint32_t, t);
  t = bf16x2{(__bf16)w[6], (__bf16)w[7]}; r.w = __builtin_bit_cast(uint32_t, t);
  return r;
}

template <typename TY>
__device__ __forceinline__ void store1(void* y, int64_t i, float v) {
  if constexpr (sizeof(TY) == 4) {
    ((float*)y)[i] = v;
  } else {
    ((uint16_t*)y)[i] = (uint16_t)f32_to_bf16_bits(v);
  }
}

}  // namespace

template <typename TS, typename TY>
__global__ __launch_bounds__(256, 1) void k_w4a16_gemm(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, const uint8_t* __restrict__ packed,
    const void* __restrict__ scales, const void* __restrict__ zeros, int64_t N, int g,
    void* __restrict__ y, int tiles_m, int tiles_n) {
  typedef typename GS<TS>::T R;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* sA = smem;                 // [2][BM][LDS_ROW]
  uint16_t* sB = smem + 2 * A_STAGE;   // [2][BN][LDS_ROW]

  // ---- tile of this workgroup -------------------------------------------
  const int bid = blockIdx.x;
  int tm, tn;
  if (tiles_m % 8 == 0) {  // XCD x (= bid mod 8) keeps M blocks x, x+8, ...
    const int xcd = bid & 7, j = bid >> 3, per = tiles_m >> 3;
    tm = xcd + 8 * (j % per);
    tn = j / per;
  } else {
    tm = bid % tiles_m;
    tn = bid / tiles_m;
  }
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // wave block: rows wm*128, cols wn*64

  // ---- global -> register assignment ----------------------------------------
  // x: 8 rounds of 32 rows; lane (t & 7) takes 16 bytes of a row's 128.
  const int xr = tid >> 3, xc = tid & 7;
  const u32x4* xp[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    int64_t row = m0 + xr + 32 * r;
    row = row < M ? row : M - 1;
    xp[r] = (const u32x4*)(x + row * K) + xc;  // + 8 * kstep
  }
  // W: 2 lanes per row, 16 bytes (32 codes) each.
  const int wr = tid >> 1, wh = tid & 1;
  int64_t wrow = n0 + wr;
  wrow = wrow < N ? wrow : N - 1;
  const u32x4* wp = (const u32x4*)(packed + wrow * (K / 2)) + wh;  // + 2 * kstep
  const int64_t ng = K / g;
  const R* sp = (const R*)scales + wrow * ng;
  const R* zp = (const R*)zeros + wrow * ng;

  const int nks = (int)(K / BK);
  u32x4 xv[8], wv;
  R sv, zv;
  auto gload = [&](int ks) {
#pragma unroll
    for (int r = 0; r < 8; ++r) xv[r] = xp[r][8 * ks];
    wv = wp[2 * ks];
    const int gi = (ks * BK + 32 * wh) / g;
    sv = sp[gi];
    zv = zp[gi];
  };
  auto lstore = [&](int stage) {
    uint16_t* a = sA + stage * A_STAGE;
#pragma unroll
    for (int r = 0; r < 8; ++r) *(u32x4*)(a + (xr + 32 * r) * LDS_ROW + 8 * xc) = xv[r];
    const float s = GS<TS>::f(sv);
    const float b = -GS<TS>::f(zv) * s;
    uint16_t* bp = sB + stage * B_STAGE + wr * LDS_ROW + 32 * wh;
    *(u32x4*)(bp + 0) = dequant8(wv.x, s, b);
    *(u32x4*)(bp + 8) = dequant8(wv.y, s, b);
    *(u32x4*)(bp + 16) = dequant8(wv.z, s, b);
    *(u32x4*)(bp + 24) = dequant8(wv.w, s, b);
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  gload(0);
  lstore(0);
  __syncthreads();

  const int l32 = lane & 31, lk = 8 * (lane >> 5);
  for (int ks = 0; ks < nks; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < nks) gload(ks + 1);
    const uint16_t* a = sA + cur * A_STAGE + (wm * 128 + l32) * LDS_ROW + lk;
    const uint16_t* b = sB + cur * B_STAGE + (wn * 64 + l32) * LDS_ROW + lk;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[4], bfr[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = *(const bf16x8*)(a + 32 * i * LDS_ROW + 16 * kk);
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[j] = *(const bf16x8*)(b + 32 * j * LDS_ROW + 16 * kk);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (ks + 1 < nks) lstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds rows 8(r/4) + 4(lane/32) + r%4, column lane%32 --
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + wn * 64 + 32 * j + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 128 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < M && n < N) store1<TY>(y, m * N + n, acc[i][j][r]);
      }
    }
}

bool gemm_fits(int64_t m, int64_t k, int g) { return m > 16 && k % BK == 0 && g % 32 == 0; }

template <typename TS, typename TY>
static hipError_t gemm_go(const uint16_t* x, int64_t m, int64_t k, const uint8_t* packed,
                          const void* scales, const void* zeros, int64_t n, int g, void* y,
                          hipStream_t st) {
  static bool attr_set = false;  // LDS above the 64 KB default
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)k_w4a16_gemm<TS, TY>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kGemmLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int tiles_m = (int)((m + BM - 1) / BM), tiles_n = (int)((n + BN - 1) / BN);
  const dim3 grid((unsigned)(tiles_m * tiles_n));
  k_w4a16_gemm<TS, TY><<<grid, 256, kGemmLds, st>>>(x, m, k, packed, scales, zeros, n, g, y,
                                                   tiles_m, tiles_n);
  return hipGetLastError();
}

hipError_t launch_w4a16_gemm(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                             const void* scales, const void* zeros, int sz_dtype, int64_t n,
                             int g, void* y, int y_dtype, hipStream_t st) {
  const uint16_t* xb = (const uint16_t*)x;
  if (sz_dtype == W4_F16) {
    if (y_dtype == W4_F32) return gemm_go<_Float16, float>(xb, m, k, packed, scales, zeros, n, g, y, st);
    return gemm_go<_Float16, __bf16>(xb, m, k, packed, scales, zeros, n, g, y, st);
  }
  if (y_dtype == W4_F32) return gemm_go<float, float>(xb, m, k, packed, scales, zeros, n, g, y, st);
  return gemm_go<float, __bf16>(xb, m, k, packed, scales, zeros, n, g, y, st);
}

}  // namespace w4
