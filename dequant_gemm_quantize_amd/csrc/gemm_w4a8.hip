// Fused W4A8 GEMM for many tokens: INT8 activations (per-token scale) times
// INT4 weights (per-group scale and zero-point) on the int8 MFMA units.
//
// Math ("Hands-on Build Guide: Group-wise INT4 Weight-only Quantization with
// Per-channel Scales", Step 5, with the weight dequantization of "From
// Scratch: Building a GPTQ INT4 Quantizer in Pure Python", Step 4):
//   y[m, n] = s_a[m] * sum_g s[n, g] * sum_{k in g} xq[m, k] * (q[n, k] - zp[n, g]).
// The inner sums are exact in int32 (|xq| <= 128, |q - zp| <= 15).  Each
// K step of 128 columns lies inside one group (group sizes are multiples of
// 128), so the int32 accumulators of a step are converted to fp32 and added
// into the fp32 accumulators with that group's scale; the token scale is
// applied once at the end.
//
// Tiling.  Workgroup tile BM (M) x 128 (N), K steps of 128, BM / 32 waves in
// a (BM / 64) x 2 arrangement, each a 64 x 64 output block (2 x 2 tiles of
// v_mfma_i32_32x32x32_i8).  BM = 256 above 128 tokens; BM = 128 up to 128
// tokens, where two workgroups share a CU, one wave of each per SIMD, and
// the two drift apart between their barriers, so one workgroup's conversions
// overlap the other's MFMAs ([28672, 8192] at 32 / 64 / 128 tokens: 76 / 80 /
// 82 us against 100 / 104 / 105 us with BM = 256, which is faster from 256
// tokens on: 114 against 126 us).  The weight tile is turned into int8 (q - zp) once
// per workgroup while it is written to LDS; the activation tile is copied as
// is.  Both are double-buffered in LDS; the global loads of x run one K step
// ahead and those of the weights two, held in registers.
// Split K (a caller's workspace, shapes with fewer than 128 tiles): workgroup
// (tile, s) covers a contiguous range of K steps and writes its token-scaled
// float32 partial tile to the workspace; k_splitk_reduce adds the splits in
// order and rounds once.  A split boundary falls between K steps, so every
// integer sum stays exact.
#include <type_traits>

#include "w4_common.h"
#include "w4_internal.h"

namespace w4 {

namespace {

constexpr int BN = 128, BK = 128;
constexpr int ROW = BK + 16;            // bytes per LDS row (+16 bytes of padding)
constexpr int B_STAGE = BN * ROW;       // bytes
constexpr int S_STAGE = BN * 4;         // fp32 group scales of the tile's rows
// Shape constants of a workgroup tile of BM (128 or 256) tokens.
template <int BM_> struct W8Tile {
  static constexpr int BM = BM_;
  static constexpr int NT = 2 * BM;            // threads: BM / 64 x 2 waves of 64 x 64 outputs
  static constexpr int WB = BN * BK / 2 / NT;  // packed weight bytes per thread and K step
  static constexpr int WL = BK / 2 / WB;       // lanes per weight row
  static constexpr int A_STAGE = BM * ROW;     // bytes
  static constexpr size_t lds = (size_t)2 * (A_STAGE + B_STAGE + S_STAGE);
};

template <typename TS> struct G8;
template <> struct G8<_Float16> {
  typedef uint16_t T;
  __device__ static float f(T v) { return (float)__builtin_bit_cast(_Float16, v); }
};
template <> struct G8<float> {
  typedef uint32_t T;
  __device__ static float f(T v) { return __uint_as_float(v); }
};

// 8 codes of a packed word -> 8 int8 values q - zp in column order, given
// c = 0x80808080 - zp * 0x01010101: per byte q + 128 - zp lies in [113, 143],
// so the add has no carries, and flipping bit 7 turns it into the two's
// complement byte of q - zp.
__device__ __forceinline__ u32x2 centre8(uint32_t p, uint32_t c) {
  const uint32_t lo = (p & 0x0f0f0f0fu) + c;          // codes 0, 2, 4, 6
  const uint32_t hi = ((p >> 4) & 0x0f0f0f0fu) + c;   // codes 1, 3, 5, 7
  u32x2 r;
  r.x = __builtin_amdgcn_perm(hi, lo, 0x05010400u) ^ 0x80808080u;  // 0 1 2 3
  r.y = __builtin_amdgcn_perm(hi, lo, 0x07030602u) ^ 0x80808080u;  // 4 5 6 7
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

template <typename TS, typename TY, bool G128, int BM>
__global__ __launch_bounds__(2 * BM, 256 / BM) void k_w4a8_gemm(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, int64_t M, int64_t K,
    const uint8_t* __restrict__ packed, const void* __restrict__ scales,
    const void* __restrict__ zeros, int64_t N, int g, void* __restrict__ y, int tiles_m, int tiles_n,
    int kps, float* __restrict__ part, int64_t pstride) {
  typedef typename G8<TS>::T R;
  typedef W8Tile<BM> T8;
  constexpr int NT = T8::NT, WB = T8::WB, WL = T8::WL, A_STAGE = T8::A_STAGE;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem8[];
  uint8_t* sA = smem8;                          // [2][BM][ROW]
  uint8_t* sB = smem8 + 2 * A_STAGE;            // [2][BN][ROW]
  float* sS = (float*)(smem8 + 2 * (A_STAGE + B_STAGE));  // [2][BN]

  const int bid = blockIdx.x;
  int tm, tn;
  if (tiles_m % 8 == 0) {  // XCD x (= bid mod 8) keeps M blocks x, x+8, ...
    const int xcd = bid & 7, j = bid >> 3, per = tiles_m >> 3;
    tm = xcd + 8 * (j % per);
    tn = j / per;
  } else {
    // groups of 8 N blocks x all M blocks, M blocks of one N block 8 ids
    // apart: those land on the same XCD, which then fetches that N block's
    // weights from HBM once for all M blocks (the last group may be narrower)
    const int span = 8 * tiles_m, grp = bid / span, r = bid % span;
    const int w = tiles_n - 8 * grp < 8 ? tiles_n - 8 * grp : 8;
    tm = r / w;
    tn = 8 * grp + r % w;
  }
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // wave block: rows wm*64, cols wn*64

  // x: 4 rounds of NT/8 rows; lane (t & 7) takes 16 bytes of a row's 128.
  constexpr int XRS = NT / 8;
  const int xr = tid >> 3, xc = tid & 7;
  const int8_t* xt = xq + m0 * K + 16 * xc;
  int xo[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int64_t row = m0 + xr + XRS * r;
    row = row < M ? row : M - 1;
    xo[r] = (int)((row - m0) * K);  // bytes, + 128 * kstep
  }
  // W: WL lanes per row, WB bytes (2 WB codes) each.
  const int wr = tid / WL, wql = tid % WL;
  int64_t wrow = n0 + wr;
  wrow = wrow < N ? wrow : N - 1;
  const uint8_t* wp = packed + wrow * (K / 2) + WB * wql;  // + 64 * kstep
  const int64_t ng = K / g;
  const int spg = g / BK;  // K steps per group
  const R* sp = (const R*)scales + wrow * ng;
  const R* zp = (const R*)zeros + wrow * ng;

  // x runs one K step ahead of the MFMAs, the weights (HBM) two.  Loads past
  // the last step are clamped to it, so the loop has no conditional loads.
  constexpr int WV = WB / 16;
  // Split K: workgroup (tile, s = blockIdx.y) covers K steps [ks0, nks).
  const int ks0 = (int)blockIdx.y * kps;
  const int nks_all = (int)(K / BK);
  const int nks = (nks_all - ks0 < kps ? nks_all - ks0 : kps) + ks0;  // one past the split's last step
  u32x4 xv[4];
  u32x4 wv[2][WV];
  R sv[2], zv[2];
  auto xload = [&](int ks) {
    ks = ks < nks ? ks : nks - 1;
#pragma unroll
    for (int r = 0; r < 4; ++r) xv[r] = *(const u32x4*)(xt + xo[r] + (int64_t)BK * ks);
  };
  auto wload = [&](int ks, auto stage) {
    constexpr int u = decltype(stage)::value;
    ks = ks < nks ? ks : nks - 1;
#pragma unroll
    for (int v = 0; v < WV; ++v) wv[u][v] = *(const u32x4*)(wp + (int64_t)(BK / 2) * ks + 16 * v);
    const int gi = G128 ? ks : ks / spg;
    sv[u] = sp[gi];
    zv[u] = zp[gi];
  };
  auto lstore = [&](int lstage, auto stage) {
    constexpr int u = decltype(stage)::value;
    uint8_t* a = sA + lstage * A_STAGE;
#pragma unroll
    for (int r = 0; r < 4; ++r) *(u32x4*)(a + (xr + XRS * r) * ROW + 16 * xc) = xv[r];
    const uint32_t zi = (uint32_t)G8<TS>::f(zv[u]);
    const uint32_t c = 0x80808080u - zi * 0x01010101u;
    uint8_t* bp = sB + lstage * B_STAGE + wr * ROW + 2 * WB * wql;
#pragma unroll
    for (int v = 0; v < WV; ++v) {
      const u32x2 b0 = centre8(wv[u][v].x, c), b1 = centre8(wv[u][v].y, c);
      const u32x2 b2 = centre8(wv[u][v].z, c), b3 = centre8(wv[u][v].w, c);
      *(u32x4*)(bp + 32 * v + 0) = u32x4{b0.x, b0.y, b1.x, b1.y};
      *(u32x4*)(bp + 32 * v + 16) = u32x4{b2.x, b2.y, b3.x, b3.y};
    }
    sS[lstage * BN + wr] = G8<TS>::f(sv[u]);  // the row's lanes store the same value
  };

  f32x16 acc[2][2];
  i32x16 ia[2][2];  // int32 sums of the current K step, one half (i) at a time
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc[i][j][r] = 0.0f;
        ia[i][j][r] = 0;
      }
  float sc[2] = {0.0f, 0.0f};  // group scales of this lane's two columns

  const int l32 = lane & 31, lk = 16 * (lane >> 5);
  // Half i of a K step: the MFMAs of rows 32i..32i+31 of the wave block into
  // ia[i], interleaved with the fp32 fold of the other half (1 - i), whose
  // MFMAs finished one phase earlier (the previous step's, for i = 0).  The
  // matrix cores and the vector ALU then work at the same time.
  auto half = [&](int lstage, auto hi, const i32x4 (&bfr)[2][BK / 32]) {
    constexpr int i = decltype(hi)::value;
    const uint8_t* a = sA + lstage * A_STAGE + (wm * 64 + 32 * i + l32) * ROW + lk;
    i32x4 af[BK / 32];
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) af[kk] = *(const i32x4*)(a + 32 * kk);
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        ia[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[kk], bfr[j][kk],
                                                        kk == 0 ? i32x16{} : ia[i][j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[1 - i][j][r] = fmaf(sc[j], (float)ia[1 - i][j][r], acc[1 - i][j][r]);
  };
  auto mma = [&](int lstage) {
    // The instruction order inside the step is left to the compiler's
    // single-wave small-GEMM strategy (iglp_opt 1): M = 512 222-224 ->
    // 212-214 us, M = 32..256 5-8% faster, against one MFMA per eight VALU
    // pinned with scheduling-group barriers (same box, alternating runs).
    __builtin_amdgcn_iglp_opt(1);
    const uint8_t* b = sB + lstage * B_STAGE + (wn * 64 + l32) * ROW + lk;
    i32x4 bfr[2][BK / 32];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int kk = 0; kk < BK / 32; ++kk) bfr[j][kk] = *(const i32x4*)(b + 32 * j * ROW + 32 * kk);
    half(lstage, std::integral_constant<int, 0>{}, bfr);  // folds half 1 of the previous step
    const float* ss = sS + lstage * BN + wn * 64 + l32;
    sc[0] = ss[0];
    sc[1] = ss[32];
    half(lstage, std::integral_constant<int, 1>{}, bfr);  // folds half 0 of this step
  };

  // Steps are counted from the split's first one: local step t is K step
  // ks0 + t (the loads clamp past the split's last step).
  xload(ks0 + 0);
  wload(ks0 + 0, std::integral_constant<int, 0>{});
  wload(ks0 + 1, std::integral_constant<int, 1>{});
  lstore(0, std::integral_constant<int, 0>{});
  xload(ks0 + 1);
  __syncthreads();

  // One K step: weights for ks + 2 in flight, MFMAs on buffer ks & 1, step
  // ks + 1 (x loaded by the previous step) into the other buffer, barrier,
  // then x for ks + 2.
  auto step = [&](int ks, auto stage) {
    constexpr int u = decltype(stage)::value;  // ks mod 2
    wload(ks0 + ks + 2, stage);  // register stage u: step ks's weights are in LDS
    mma(ks & 1);
    lstore((ks + 1) & 1, std::integral_constant<int, 1 - u>{});
    __syncthreads();
    xload(ks0 + ks + 2);
  };
  const int nloc = nks - ks0;  // steps of this split
  const int nmain = nloc & ~1;
  for (int ks = 0; ks < nmain; ks += 2) {
    step(ks, std::integral_constant<int, 0>{});
    step(ks + 1, std::integral_constant<int, 1>{});
  }
  if (nmain < nloc) step(nmain, std::integral_constant<int, 0>{});
  // fold half 1 of the last step
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[1][j][r] = fmaf(sc[j], (float)ia[1][j][r], acc[1][j][r]);

  // ---- epilogue: lane holds rows 8(r/4) + 4(lane/32) + r%4, column lane%32 --
  // Whole 64 x 64 blocks take the store without bounds tests (M = 512:
  // 210-213 -> 195-197 us).  Not with BM = 128: there the extra live values
  // reorder the main loop's loads, and 32 to 128 tokens got 10-20% slower.
  // With split K the token-scaled float32 partial goes to part + s * pstride
  // as [M][N]; k_splitk_reduce adds the splits and rounds once.
  float* pdst = part != nullptr ? part + (int64_t)blockIdx.y * pstride : nullptr;
  if constexpr (BM == 256) {
    const int64_t bm0 = m0 + wm * 64, bn0 = n0 + wn * 64;  // the wave's block
    if (bm0 + 64 <= M && bn0 + 64 <= N && N < (1 << 23)) {
      if (pdst != nullptr)
        store_wave_block<float, 2, true>(pdst + bm0 * N + bn0, N, lane, acc, xs + bm0);
      else
        store_wave_block<TY, 2, true>((TY*)y + bm0 * N + bn0, N, lane, acc, xs + bm0);
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t m = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (m >= M) continue;
      const float sa = xs[m];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t n = n0 + wn * 64 + 32 * j + l32;
        if (n < N) {
          if (pdst != nullptr)
            pdst[m * N + n] = sa * acc[i][j][r];
          else
            store1<TY>(y, m * N + n, sa * acc[i][j][r]);
        }
      }
    }
  }
}

bool w4a8_gemm_fits(int64_t m, int64_t k, int g) { return m > 16 && g % BK == 0 && k % BK == 0; }

// Split-K plan: shapes with fewer than 128 tiles (one GPU's 8-way column
// shard of the [28672, 8192] projection, [3584, 8192], has 28 tiles of
// 128 x 128 up to 128 tokens and 56 of 256 x 128 at 512) split K so that
// about 256 workgroups run, at least 8 K steps per split, with the float32
// partials within kSplitKMaxBytes.  Measured on the shard: 17 / 128 / 512 /
// 1024 tokens 59 / 66 / 78 / 82 -> 19 / 29 / 37 / 59 us.  The whole
// projection at 17 to 128 tokens (224 tiles) does not split: two splits there
// measured 70-76 -> 79-94 us.
struct SplitK8 {
  int bm = 256, s = 1, kps = 0;
  int64_t pstride = 0;  // floats per split's partial: M * N rounded up to a multiple of 4
  size_t bytes = 0;
};
static SplitK8 w4a8_splitk_plan(int64_t m, int64_t k, int64_t n) {
  SplitK8 p;
  p.bm = m <= 128 ? 128 : 256;
  const int64_t tiles = ((m + p.bm - 1) / p.bm) * ((n + BN - 1) / BN);
  const int64_t nks = k / BK;
  p.kps = (int)nks;
  if (tiles >= 128) return p;
  int64_t s = (256 + tiles - 1) / tiles;
  if (s > nks / 8) s = nks / 8;
  const int64_t pstride = (m * n + 3) / 4 * 4;
  const int64_t fit = (int64_t)(kSplitKMaxBytes / ((size_t)pstride * 4));
  if (s > fit) s = fit;
  if (s < 2) return p;
  p.kps = (int)((nks + s - 1) / s);
  p.s = (int)((nks + p.kps - 1) / p.kps);
  p.pstride = pstride;
  p.bytes = (size_t)p.s * (size_t)pstride * 4;
  return p;
}

size_t w4a8_gemm_workspace_bytes(int64_t m, int64_t k, int64_t n, int g) {
  if (!w4a8_gemm_fits(m, k, g)) return 0;
  const SplitK8 p = w4a8_splitk_plan(m, k, n);
  return p.s > 1 ? p.bytes : 0;
}

template <typename TS, typename TY, int BM>
static hipError_t w4a8_go_bm(const int8_t* xq, const float* xs, int64_t m, int64_t k,
                             const uint8_t* packed, const void* scales, const void* zeros, int64_t n,
                             int g, void* y, const SplitK8& p, float* part, hipStream_t st) {
  typedef W8Tile<BM> T8;
  static std::atomic<uint64_t> attr_done{0};  // LDS above the 64 KB default
  hipError_t e = once_per_device(attr_done, [] {
    for (const void* f : {(const void*)k_w4a8_gemm<TS, TY, true, BM>, (const void*)k_w4a8_gemm<TS, TY, false, BM>}) {
      hipError_t r = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)T8::lds);
      if (r != hipSuccess) return r;
    }
    return hipSuccess;
  });
  if (e != hipSuccess) return e;
  const int tiles_m = (int)((m + BM - 1) / BM), tiles_n = (int)((n + BN - 1) / BN);
  const dim3 grid((unsigned)(tiles_m * tiles_n), (unsigned)p.s);
  if (g == BK)
    k_w4a8_gemm<TS, TY, true, BM><<<grid, T8::NT, T8::lds, st>>>(xq, xs, m, k, packed, scales, zeros, n, g,
                                                                 y, tiles_m, tiles_n, p.kps, part, p.pstride);
  else
    k_w4a8_gemm<TS, TY, false, BM><<<grid, T8::NT, T8::lds, st>>>(xq, xs, m, k, packed, scales, zeros, n,
                                                                  g, y, tiles_m, tiles_n, p.kps, part,
                                                                  p.pstride);
  return hipGetLastError();
}

template <typename TS, typename TY>
static hipError_t w4a8_go(const int8_t* xq, const float* xs, int64_t m, int64_t k,
                          const uint8_t* packed, const void* scales, const void* zeros, int64_t n,
                          int g, void* y, int y_dtype, void* ws, size_t ws_bytes, hipStream_t st) {
  SplitK8 p = w4a8_splitk_plan(m, k, n);
  if (p.s > 1 && (ws == nullptr || ws_bytes < p.bytes)) {
    p.s = 1;
    p.kps = (int)(k / BK);
    p.pstride = 0;
    p.bytes = 0;
  }
  float* part = p.s > 1 ? (float*)ws : nullptr;
  const hipError_t e =
      m <= 128 ? w4a8_go_bm<TS, TY, 128>(xq, xs, m, k, packed, scales, zeros, n, g, y, p, part, st)
               : w4a8_go_bm<TS, TY, 256>(xq, xs, m, k, packed, scales, zeros, n, g, y, p, part, st);
  if (e != hipSuccess || p.s == 1) return e;
  return launch_splitk_reduce(part, p.s, m * n, p.pstride, y, y_dtype, st);
}

hipError_t launch_w4a8_gemm(const int8_t* xq, const float* xs, int64_t m, int64_t k,
                            const uint8_t* packed, const void* scales, const void* zeros,
                            int sz_dtype, int64_t n, int g, void* y, int y_dtype, void* ws,
                            size_t ws_bytes, hipStream_t st) {
  if (sz_dtype == W4_F16) {
    if (y_dtype == W4_F32)
      return w4a8_go<_Float16, float>(xq, xs, m, k, packed, scales, zeros, n, g, y, y_dtype, ws, ws_bytes, st);
    return w4a8_go<_Float16, __bf16>(xq, xs, m, k, packed, scales, zeros, n, g, y, y_dtype, ws, ws_bytes, st);
  }
  if (y_dtype == W4_F32)
    return w4a8_go<float, float>(xq, xs, m, k, packed, scales, zeros, n, g, y, y_dtype, ws, ws_bytes, st);
  return w4a8_go<float, __bf16>(xq, xs, m, k, packed, scales, zeros, n, g, y, y_dtype, ws, ws_bytes, st);
}

}  // namespace w4
