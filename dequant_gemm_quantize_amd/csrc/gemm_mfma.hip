// Prefill fused dequantize-GEMM: y = x . dequant(W)^T for many tokens (bf16
// x), bf16 MFMA with fp32 accumulation.  MFMA-bound at M = 2048.
//
// Math ("Building a From-Scratch Group-Wise INT4 Quantization Layer for
// LLaMA Weights", Step 2, with the dequantization of "From Scratch: Building
// a GPTQ INT4 Quantizer in Pure Python", Step 4): every weight tile is
// dequantized once per workgroup to bf16 as fma(q, s, -zp*s) and written to
// LDS, where it feeds v_mfma_f32_32x32x16_bf16 together with the activation
// tile.  No dequantized matrix ever reaches memory.  With fp16 scales, q*s
// and zp*s are exact in fp32 (4 + 11 significant bits), so the weight is
// RNE((q - zp) * s) with one rounding.  With fp32 scales zp*s is itself
// rounded, so a weight can differ from that by one bf16 step where the exact
// product sits at a bf16 tie; the accuracy bound of the product holds either
// way.
//
// Tiling.  Workgroup tile 256 (M) x 128 (N), K in steps of 64, both operand
// tiles double-buffered in LDS (rows padded by 16 bytes).  Eight waves (two
// per SIMD: a wave alone cannot pull LDS fast enough to feed its MFMAs) in a
// 4 x 2 arrangement, each owning a 64 x 64 block of the output: 2 x 2 MFMA
// tiles of 32 x 32, 64 fp32 accumulators per lane.  The global loads of the
// following K steps are in flight (held in registers, W4_GEMM_DEPTH steps
// deep) while the current one runs on the MFMA units.
// Tiles are numbered so that consecutive workgroups (which the dispatcher
// spreads over the 8 XCDs) share an N block and each XCD keeps working on
// the same M block of x, which then stays in that XCD's L2.
#include <type_traits>

#include "w4_common.h"
#include "w4_internal.h"

namespace w4 {

namespace {

#ifndef W4_GEMM_DEPTH
#define W4_GEMM_DEPTH 4
#endif
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
__global__ __launch_bounds__(512, 1) void k_w4a16_gemm(
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
  const int wm = wave >> 1, wn = wave & 1;  // wave block: rows wm*64, cols wn*64

  // ---- global -> register assignment ----------------------------------------
  // x: 4 rounds of 64 rows; lane (t & 7) takes 16 bytes of a row's 128.
  const int xr = tid >> 3, xc = tid & 7;
  const uint16_t* xt = x + m0 * K;  // tile base (uniform); per-lane offsets below
  int xo[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int64_t row = m0 + xr + 64 * r;
    row = row < M ? row : M - 1;
    xo[r] = (int)((row - m0) * K) + 8 * xc;  // elements, + 64 * kstep
  }
  // W: 4 lanes per row, 8 bytes (16 codes) each.
  const int wr = tid >> 2, wq4 = tid & 3;
  int64_t wrow = n0 + wr;
  wrow = wrow < N ? wrow : N - 1;
  const uint32_t* wp = (const uint32_t*)(packed + wrow * (K / 2)) + 2 * wq4;  // + 8 * kstep
  const int64_t ng = K / g;
  const R* sp = (const R*)scales + wrow * ng;
  const R* zp = (const R*)zeros + wrow * ng;

  // Global data runs D K-steps ahead of the MFMAs, in D register stages
  // (stage = K-step mod D): loads for step ks + D are issued while step ks
  // computes, and step ks + 1 is dequantized into the other LDS buffer after
  // it.  Every wait is then for loads issued D - 1 steps earlier.
  constexpr int D = W4_GEMM_DEPTH;
  const int nks = (int)(K / BK);
  u32x4 xv[D][4];
  u32x2 wv[D];
  R sv[D], zv[D];
  // Loads past the last K step are clamped to it (a few redundant loads)
  // so that the main loop has no conditional loads: the compiler can then
  // wait for exactly the stage it needs instead of for every load.
  auto gload = [&](int ks, auto stage) {
    constexpr int u = decltype(stage)::value;
    ks = ks < nks ? ks : nks - 1;
#pragma unroll
    for (int r = 0; r < 4; ++r) xv[u][r] = *(const u32x4*)(xt + xo[r] + 64 * ks);
    wv[u] = *(const u32x2*)(wp + 8 * ks);
    const int gi = (ks * BK + 16 * wq4) / g;
    sv[u] = sp[gi];
    zv[u] = zp[gi];
  };
  auto lstore = [&](int lstage, auto stage) {
    constexpr int u = decltype(stage)::value;
    uint16_t* a = sA + lstage * A_STAGE;
#pragma unroll
    for (int r = 0; r < 4; ++r) *(u32x4*)(a + (xr + 64 * r) * LDS_ROW + 8 * xc) = xv[u][r];
    const float s = GS<TS>::f(sv[u]);
    const float b = -GS<TS>::f(zv[u]) * s;
    uint16_t* bp = sB + lstage * B_STAGE + wr * LDS_ROW + 16 * wq4;
    *(u32x4*)(bp + 0) = dequant8(wv[u].x, s, b);
    *(u32x4*)(bp + 8) = dequant8(wv[u].y, s, b);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int l32 = lane & 31, lk = 8 * (lane >> 5);
  auto mma = [&](int lstage) {
    const uint16_t* a = sA + lstage * A_STAGE + (wm * 64 + l32) * LDS_ROW + lk;
    const uint16_t* b = sB + lstage * B_STAGE + (wn * 64 + l32) * LDS_ROW + lk;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = *(const bf16x8*)(a + 32 * i * LDS_ROW + 16 * kk);
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[j] = *(const bf16x8*)(b + 32 * j * LDS_ROW + 16 * kk);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  // prologue: steps 0 .. D-1 in flight, step 0 in LDS buffer 0
  gload(0, std::integral_constant<int, 0>{});
  if constexpr (D > 1) gload(1, std::integral_constant<int, 1 % D>{});
  if constexpr (D > 2) gload(2, std::integral_constant<int, 2 % D>{});
  if constexpr (D > 3) gload(3, std::integral_constant<int, 3 % D>{});
  lstore(0, std::integral_constant<int, 0>{});
  __syncthreads();

  // One K step, unconditional: loads for ks + D, MFMAs on buffer ks & 1,
  // dequantize step ks + 1 into the other buffer (past the end this writes
  // the idle buffer, which is never read), barrier.
  auto step = [&](int ks, auto stage) {
    constexpr int u = decltype(stage)::value;  // ks mod D
    gload(ks + D, stage);  // reuses register stage u: step ks is already in LDS
    mma(ks & 1);
    lstore((ks + 1) & 1, std::integral_constant<int, (u + 1) % D>{});
    __syncthreads();
  };
  const int nmain = nks - nks % D;
  for (int ks = 0; ks < nmain; ks += D) {
    step(ks, std::integral_constant<int, 0>{});
    if constexpr (D > 1) step(ks + 1, std::integral_constant<int, 1 % D>{});
    if constexpr (D > 2) step(ks + 2, std::integral_constant<int, 2 % D>{});
    if constexpr (D > 3) step(ks + 3, std::integral_constant<int, 3 % D>{});
  }
  // tail: the remaining nks % D steps (register stage of step ks is ks mod D)
  if (nmain < nks) step(nmain, std::integral_constant<int, 0>{});
  if constexpr (D > 1) if (nmain + 1 < nks) step(nmain + 1, std::integral_constant<int, 1 % D>{});
  if constexpr (D > 2) if (nmain + 2 < nks) step(nmain + 2, std::integral_constant<int, 2 % D>{});

  // ---- epilogue: lane holds rows 8(r/4) + 4(lane/32) + r%4, column lane%32 --
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + wn * 64 + 32 * j + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < M && n < N) store1<TY>(y, m * N + n, acc[i][j][r]);
      }
    }
}

bool gemm_fits(int64_t m, int64_t k, int g) { return m > 16 && k % BK == 0 && g % 32 == 0; }

template <typename TS, typename TY>
static hipError_t gemm_go(const uint16_t* x, int64_t m, int64_t k, const uint8_t* packed,
                          const void* scales, const void* zeros, int64_t n, int g, void* y,
                          hipStream_t st) {
  static std::atomic<uint64_t> attr_done{0};  // LDS above the 64 KB default
  hipError_t e = once_per_device(attr_done, [] {
    return hipFuncSetAttribute((const void*)k_w4a16_gemm<TS, TY>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)kGemmLds);
  });
  if (e != hipSuccess) return e;
  const int tiles_m = (int)((m + BM - 1) / BM), tiles_n = (int)((n + BN - 1) / BN);
  const dim3 grid((unsigned)(tiles_m * tiles_n));
  k_w4a16_gemm<TS, TY><<<grid, 512, kGemmLds, st>>>(x, m, k, packed, scales, zeros, n, g, y,
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
