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
constexpr int BM = 256, BN = 128, BK = 64;  // BN: the split-K tiles; wide tiles take 192
constexpr int LDS_ROW = BK + 8;  // bf16 elements per LDS row (+16 bytes of padding)
constexpr int A_STAGE = BM * LDS_ROW;
// LDS of a workgroup with N tiles of 64 * NJ columns (NJ = 2: 128, NJ = 3: 192)
constexpr size_t gemm_lds(int nj) { return (size_t)2 * (A_STAGE + 64 * nj * LDS_ROW) * 2; }

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
// w = RNE(fma(q, s, b)) with b = -zp * s.  Each code is converted straight
// from its byte of the masked word (v_cvt_f32_ubyte0..3).
__device__ __forceinline__ u32x4 dequant8(uint32_t p, float s, float b) {
  uint32_t lo = p & 0x0f0f0f0fu;         // codes 0, 2, 4, 6
  uint32_t hi = (p >> 4) & 0x0f0f0f0fu;  // codes 1, 3, 5, 7
  // The empty asm emits nothing; it hides the masks from the combiner, which
  // would otherwise fold each byte's mask into a v_bfe_u32 ahead of the
  // conversion instead of converting the byte in place.
  asm("" : "+v"(lo), "+v"(hi));
  float w[8];
  w[0] = fmaf((float)(uint8_t)lo, s, b);
  w[1] = fmaf((float)(uint8_t)hi, s, b);
  w[2] = fmaf((float)(uint8_t)(lo >> 8), s, b);
  w[3] = fmaf((float)(uint8_t)(hi >> 8), s, b);
  w[4] = fmaf((float)(uint8_t)(lo >> 16), s, b);
  w[5] = fmaf((float)(uint8_t)(hi >> 16), s, b);
  w[6] = fmaf((float)(lo >> 24), s, b);
  w[7] = fmaf((float)(hi >> 24), s, b);
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

// G64: g % 64 == 0, so a K step lies in one group, the same for every
// lane: its index is umulhi(ks, gmagic) with gmagic = ceil(2^32 / (g / 64)),
// or ks itself when g = 64 (gmagic = 0: 2^32 does not fit).
// Otherwise each lane's 16 columns lie in one group (g % 32 == 0): index
// umulhi(c16, gmagic), c16 = the 16-column piece, gmagic = ceil(2^32 /
// (g / 16)).  Both quotients are exact while the dividend times the divisor
// stays below 2^32, which gemm_fits guarantees.
// Split K: workgroup (tile, s = blockIdx.y) covers K steps [s * kps,
// min(nks, (s + 1) * kps)) and, when `part` is set, writes its float32 partial
// tile to part + s * pstride as [M][N] (y is then unused; pstride is M * N
// rounded up to a multiple of 4); k_splitk_reduce adds the splits.
// NJ: the workgroup tile is BM x 64 NJ (NJ = 2 or 3); each wave owns 64 x
// 32 NJ of it (2 x NJ MFMA tiles).  Weight rows are loaded and dequantized
// by BK / CPL lanes each, CPL = 16 codes (NJ = 2: all 512 threads) or 32
// codes (NJ = 3: the first 384 threads, six whole waves).
template <typename TS, typename TY, bool G64, int NJ>
__global__ __launch_bounds__(512, 1) void k_w4a16_gemm(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, const uint8_t* __restrict__ packed,
    const void* __restrict__ scales, const void* __restrict__ zeros, int64_t N, int64_t ng,
    uint32_t gmagic, void* __restrict__ y, int tiles_m, int tiles_n, int kps,
    float* __restrict__ part, int64_t pstride) {
  typedef typename GS<TS>::T R;
  constexpr int BNt = 64 * NJ;              // tile columns
  constexpr int B_STAGE = BNt * LDS_ROW;
  constexpr int CPL = NJ == 2 ? 16 : 32;    // codes per weight lane and K step
  constexpr int LPR = BK / CPL;             // lanes per weight row
  constexpr int WTHR = BNt * LPR;           // threads that load weights (512 or 384)
  typedef typename std::conditional<CPL == 16, u32x2, u32x4>::type WV;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* sA = smem;                 // [2][BM][LDS_ROW]
  uint16_t* sB = smem + 2 * A_STAGE;   // [2][BNt][LDS_ROW]

  // ---- tile of this workgroup -------------------------------------------
  const int bid = blockIdx.x;
  int tm, tn;
  if (tiles_m % 8 == 0) {  // XCD x (= bid mod 8) keeps M blocks x, x+8, ...
    const int xcd = bid & 7, j = bid >> 3, per = tiles_m >> 3;
    tm = xcd + 8 * (j % per);
    tn = j / per;
  } else {
    // consecutive ids cycle through the M blocks, so with an even number of
    // them each XCD keeps to every other M block of x (measured faster here
    // than grouping an N block's M blocks on one XCD: x is re-read every K
    // step, the weights once per M block)
    tm = bid % tiles_m;
    tn = bid / tiles_m;
  }
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BNt;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // wave block: rows wm*64, cols wn*32*NJ

  // ---- global -> register assignment ----------------------------------------
  // Every address is a uniform base (advanced by the K step) plus a fixed
  // 32-bit lane offset.  Rows past M or N repeat the last row.
  // x: 4 rounds of 64 rows; lane (t & 7) takes 16 bytes of a row's 128.
  // Round r's base row is min(m0 + 64 r, M - 1), so lane offsets are >= 0
  // and below 64 rows of K bf16 (< 2^30 bytes).
  const int xr = tid >> 3, xc = tid & 7;
  __amdgpu_buffer_rsrc_t xrs[4];
  uint32_t xo[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t rb = m0 + 64 * r < M ? m0 + 64 * r : M - 1;
    const int64_t row = m0 + xr + 64 * r < M ? m0 + xr + 64 * r : M - 1;
    xrs[r] = buf_rsrc((const char*)x + rb * K * 2);
    xo[r] = (uint32_t)((row - rb) * K * 2) + 16u * (uint32_t)xc;
  }
  // W: LPR lanes per row, CPL / 2 bytes each; offsets below 192 rows of
  // K/2 bytes (< 2^30).  Scales and zeros: the tile's rows of K/g.
  const bool wact = tid < WTHR;  // wave-uniform (WTHR is a multiple of 64)
  const int wr = wact ? tid / LPR : 0, wq4 = tid % LPR;
  const int64_t wrow = n0 + wr < N ? n0 + wr : N - 1;
  const __amdgpu_buffer_rsrc_t wrs = buf_rsrc(packed + n0 * (K / 2));
  const uint32_t wo = (uint32_t)((wrow - n0) * (K / 2)) + (uint32_t)(CPL / 2) * (uint32_t)wq4;
  const __amdgpu_buffer_rsrc_t srs = buf_rsrc((const R*)scales + n0 * ng);
  const __amdgpu_buffer_rsrc_t zrs = buf_rsrc((const R*)zeros + n0 * ng);
  const uint32_t so = (uint32_t)((wrow - n0) * ng) * (uint32_t)sizeof(R);  // bytes

  // Global data runs D K-steps ahead of the MFMAs, in D register stages
  // (stage = K-step mod D): loads for step ks + D are issued while step ks
  // computes, and step ks + 1 is dequantized into the other LDS buffer after
  // it.  Every wait is then for loads issued D - 1 steps earlier.
  constexpr int D = W4_GEMM_DEPTH;
  const int ks0 = (int)blockIdx.y * kps;  // first K step of this split
  const int nks_all = (int)(K / BK);
  const int nks = (nks_all - ks0 < kps ? nks_all - ks0 : kps) + ks0;  // one past the last step
  u32x4 xv[D][4];
  WV wv[D];
  R sv[D], zv[D];
  // Loads past the last K step are clamped to it (a few redundant loads)
  // so that the main loop has no conditional loads: the compiler can then
  // wait for exactly the stage it needs instead of for every load.
  auto gload = [&](int ks, auto stage) {
    constexpr int u = decltype(stage)::value;
    ks = ks < nks ? ks : nks - 1;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      xv[u][r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs[r], xo[r], ks * (2 * BK), 0));
    if (!wact) return;
    if constexpr (CPL == 16)
      wv[u] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(wrs, wo, ks * (BK / 2), 0));
    else
      wv[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, wo, ks * (BK / 2), 0));
    uint32_t vo = so, go = 0;  // group offset: uniform (G64) or per lane
    if constexpr (G64) {
      go = (gmagic ? __umulhi((uint32_t)ks, gmagic) : (uint32_t)ks) * (uint32_t)sizeof(R);
    } else {
      const uint32_t piece = (uint32_t)(ks * LPR + wq4);  // CPL-column piece of the row
      vo += (gmagic ? __umulhi(piece, gmagic) : piece) * (uint32_t)sizeof(R);
    }
    if constexpr (sizeof(R) == 2) {
      sv[u] = __builtin_amdgcn_raw_buffer_load_b16(srs, vo, go, 0);
      zv[u] = __builtin_amdgcn_raw_buffer_load_b16(zrs, vo, go, 0);
    } else {
      sv[u] = __builtin_amdgcn_raw_buffer_load_b32(srs, vo, go, 0);
      zv[u] = __builtin_amdgcn_raw_buffer_load_b32(zrs, vo, go, 0);
    }
  };
  auto lstore = [&](int lstage, auto stage) {
    constexpr int u = decltype(stage)::value;
    uint16_t* a = sA + lstage * A_STAGE;
#pragma unroll
    for (int r = 0; r < 4; ++r) *(u32x4*)(a + (xr + 64 * r) * LDS_ROW + 8 * xc) = xv[u][r];
    if (!wact) return;
    const float s = GS<TS>::f(sv[u]);
    const float b = -GS<TS>::f(zv[u]) * s;
    uint16_t* bp = sB + lstage * B_STAGE + wr * LDS_ROW + CPL * wq4;
#pragma unroll
    for (int t = 0; t < CPL / 8; ++t) *(u32x4*)(bp + 8 * t) = dequant8(wv[u][t], s, b);
  };

  f32x16 acc[2][NJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int l32 = lane & 31, lk = 8 * (lane >> 5);
  auto mma = [&](int lstage) {
    // The compiler's interleaving of the fragment reads with the MFMAs
    // (strategy 1 of __builtin_amdgcn_iglp_opt): Wb M = 2048 234-238 ->
    // 229-233 us, Wd 220-223 -> 211-217 us, Wb M = 512 80-82 -> 73-76 us
    // (same box, alternating runs).
    __builtin_amdgcn_iglp_opt(1);
    const uint16_t* a = sA + lstage * A_STAGE + (wm * 64 + l32) * LDS_ROW + lk;
    const uint16_t* b = sB + lstage * B_STAGE + (wn * 32 * NJ + l32) * LDS_ROW + lk;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 af[2], bfr[NJ];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = *(const bf16x8*)(a + 32 * i * LDS_ROW + 16 * kk);
#pragma unroll
      for (int j = 0; j < NJ; ++j) bfr[j] = *(const bf16x8*)(b + 32 * j * LDS_ROW + 16 * kk);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  // Steps are counted from this split's first one: local step t is K step
  // ks0 + t (gload clamps past the split's last step, whose loads are never
  // used).
  // prologue: steps 0 .. D-1 in flight, step 0 in LDS buffer 0
  gload(ks0 + 0, std::integral_constant<int, 0>{});
  if constexpr (D > 1) gload(ks0 + 1, std::integral_constant<int, 1 % D>{});
  if constexpr (D > 2) gload(ks0 + 2, std::integral_constant<int, 2 % D>{});
  if constexpr (D > 3) gload(ks0 + 3, std::integral_constant<int, 3 % D>{});
  lstore(0, std::integral_constant<int, 0>{});
  __syncthreads();

  // One K step, unconditional: loads for ks + D, MFMAs on buffer ks & 1,
  // dequantize step ks + 1 into the other buffer (past the end this writes
  // the idle buffer, which is never read), barrier.
  auto step = [&](int ks, auto stage) {
    constexpr int u = decltype(stage)::value;  // ks mod D
    gload(ks0 + ks + D, stage);  // reuses register stage u: step ks is already in LDS
    mma(ks & 1);
    lstore((ks + 1) & 1, std::integral_constant<int, (u + 1) % D>{});
    __syncthreads();
  };
  const int nloc = nks - ks0;  // steps of this split
  const int nmain = nloc - nloc % D;
  for (int ks = 0; ks < nmain; ks += D) {
    step(ks, std::integral_constant<int, 0>{});
    if constexpr (D > 1) step(ks + 1, std::integral_constant<int, 1 % D>{});
    if constexpr (D > 2) step(ks + 2, std::integral_constant<int, 2 % D>{});
    if constexpr (D > 3) step(ks + 3, std::integral_constant<int, 3 % D>{});
  }
  // tail: the remaining nloc % D steps (register stage of step ks is ks mod D)
  if (nmain < nloc) step(nmain, std::integral_constant<int, 0>{});
  if constexpr (D > 1) if (nmain + 1 < nloc) step(nmain + 1, std::integral_constant<int, 1 % D>{});
  if constexpr (D > 2) if (nmain + 2 < nloc) step(nmain + 2, std::integral_constant<int, 2 % D>{});

  // ---- epilogue: lane holds rows 8(r/4) + 4(lane/32) + r%4, column lane%32 --
  const int64_t bm0 = m0 + wm * 64, bn0 = n0 + wn * 32 * NJ;  // the wave's block
  if (bm0 + 64 <= M && bn0 + 32 * NJ <= N && N < (1 << 23)) {
    if (part != nullptr)
      store_wave_block<float, NJ, false>(part + (int64_t)blockIdx.y * pstride + bm0 * N + bn0, N, lane, acc,
                                         nullptr);
    else
      store_wave_block<TY, NJ, false>((TY*)y + bm0 * N + bn0, N, lane, acc, nullptr);
    return;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t n = n0 + wn * 32 * NJ + 32 * j + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < M && n < N) {
          if (part != nullptr)
            part[(int64_t)blockIdx.y * pstride + m * N + n] = acc[i][j][r];
          else
            store1<TY>(y, m * N + n, acc[i][j][r]);
        }
      }
    }
}

// y[i] = sum over s = 0 .. S-1, in that order, of part[s * pstride + i]
// (float32), rounded once to y's type; 4 consecutive outputs per thread
// (pstride % 4 == 0 keeps every 16-byte load aligned; the last group of
// fewer than 4 outputs is added element by element).
template <typename TY>
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ part, int S, int64_t MN,
                                                       int64_t pstride, void* __restrict__ y) {
  const int64_t i4 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i4 >= MN) return;
  if (i4 + 4 <= MN) {
    f32x4 a = *(const f32x4*)(part + i4);
    for (int s = 1; s < S; ++s) a += *(const f32x4*)(part + (int64_t)s * pstride + i4);
#pragma unroll
    for (int j = 0; j < 4; ++j) store1<TY>(y, i4 + j, a[j]);
  } else {
    for (int64_t i = i4; i < MN; ++i) {
      float a = part[i];
      for (int s = 1; s < S; ++s) a += part[(int64_t)s * pstride + i];
      store1<TY>(y, i, a);
    }
  }
}

// The group index of a K step (g % 64 == 0) or of a 16-column piece is an
// exact magic-number quotient while dividend x divisor < 2^32: K/64 * g/64
// or K/16 * g/16 below 2^32.  Larger K * g go to the general kernel.
bool gemm_fits(int64_t m, int64_t k, int g) {
  if (!(m > 16 && k % BK == 0 && g % 32 == 0)) return false;
  return g % 64 == 0 ? (k / 64) * (g / 64) < ((int64_t)1 << 32) : (k / 16) * (g / 16) < ((int64_t)1 << 32);
}

// ceil(2^32 / d) for d >= 2; 0 for d = 1 (the kernels then take the dividend itself).
static uint32_t magic_ceil(uint32_t d) { return d < 2 ? 0u : (uint32_t)((((uint64_t)1 << 32) + d - 1) / d); }

// Split-K plan: shapes whose 256 x 128 tiles fill fewer than half of the 256
// CUs (the [4096, 11008] down projection below 513 tokens has 32 or 64)
// split K so that about 256 workgroups run, at least 8 K steps each, with the
// float32 partials within kSplitKMaxBytes.
struct SplitK {
  int s = 1, kps = 0;
  int64_t pstride = 0;  // floats per split's partial: M * N rounded up to a multiple of 4
  size_t bytes = 0;
};
static SplitK splitk_plan(int64_t m, int64_t k, int64_t n) {
  SplitK p;
  const int64_t tiles = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
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

size_t gemm_workspace_bytes(int64_t m, int64_t k, int64_t n, int g) {
  if (!gemm_fits(m, k, g)) return 0;
  const SplitK p = splitk_plan(m, k, n);
  return p.s > 1 ? p.bytes : 0;
}

// Tiles 192 wide move 18% fewer LDS bytes per flop (the kernel's limit at
// large M) and take 1.36x as long each (measured on [11008, 4096] at
// M = 2048: 115.5 us per round of 256 wide tiles against 85 us for 128-wide
// ones); they are chosen when their rounds of 256 workgroups, weighted 1.36,
// come out below the 128-wide tiles' rounds.
#ifndef W4_GEMM_WIDE
#define W4_GEMM_WIDE 1
#endif
static bool wide_tiles(int64_t m, int64_t n) {
  if (!W4_GEMM_WIDE) return false;
  const int64_t tm = (m + BM - 1) / BM;
  const int64_t r128 = (tm * ((n + 127) / 128) + 255) / 256;
  const int64_t r192 = (tm * ((n + 191) / 192) + 255) / 256;
  return (double)r192 * 1.36 < (double)r128;
}

template <typename TS, typename TY, bool G64, int NJ>
static hipError_t gemm_launch(const uint16_t* x, int64_t m, int64_t k, const uint8_t* packed,
                              const void* scales, const void* zeros, int64_t n, int g, void* y,
                              const SplitK& p, float* part, hipStream_t st) {
  static std::atomic<uint64_t> attr_done{0};  // LDS above the 64 KB default
  hipError_t e = once_per_device(attr_done, [] {
    return hipFuncSetAttribute((const void*)k_w4a16_gemm<TS, TY, G64, NJ>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)gemm_lds(NJ));
  });
  if (e != hipSuccess) return e;
  const int tiles_m = (int)((m + BM - 1) / BM), tiles_n = (int)((n + 64 * NJ - 1) / (64 * NJ));
  // the quotient of a K step (g % 64 == 0) or of a lane's CPL-column piece
  const int cpl = NJ == 2 ? 16 : 32;
  const uint32_t gm = magic_ceil((uint32_t)(G64 ? g / 64 : g / cpl));
  const dim3 grid((unsigned)(tiles_m * tiles_n), (unsigned)p.s);
  k_w4a16_gemm<TS, TY, G64, NJ><<<grid, 512, gemm_lds(NJ), st>>>(x, m, k, packed, scales, zeros, n, k / g, gm,
                                                                y, tiles_m, tiles_n, p.kps, part, p.pstride);
  return hipGetLastError();
}

template <typename TS, typename TY, bool G64>
static hipError_t gemm_go(const uint16_t* x, int64_t m, int64_t k, const uint8_t* packed,
                          const void* scales, const void* zeros, int64_t n, int g, void* y,
                          void* ws, size_t ws_bytes, hipStream_t st) {
  SplitK p = splitk_plan(m, k, n);
  if (p.s > 1 && (ws == nullptr || ws_bytes < p.bytes)) p = SplitK{1, (int)(k / BK), 0, 0};
  float* part = p.s > 1 ? (float*)ws : nullptr;
  hipError_t e;
  if (p.s == 1 && wide_tiles(m, n))
    e = gemm_launch<TS, TY, G64, 3>(x, m, k, packed, scales, zeros, n, g, y, p, part, st);
  else
    e = gemm_launch<TS, TY, G64, 2>(x, m, k, packed, scales, zeros, n, g, y, p, part, st);
  if (e != hipSuccess) return e;
  if (p.s > 1) {
    const int64_t mn = m * n;
    const dim3 rgrid((unsigned)((mn + 1023) / 1024));
    k_splitk_reduce<TY><<<rgrid, 256, 0, st>>>(part, p.s, mn, p.pstride, y);
  }
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float* part, int S, int64_t mn, int64_t pstride, void* y,
                                int y_dtype, hipStream_t st) {
  const dim3 rgrid((unsigned)((mn + 1023) / 1024));
  if (y_dtype == W4_F32)
    k_splitk_reduce<float><<<rgrid, 256, 0, st>>>(part, S, mn, pstride, y);
  else
    k_splitk_reduce<__bf16><<<rgrid, 256, 0, st>>>(part, S, mn, pstride, y);
  return hipGetLastError();
}

template <typename TS, typename TY>
static hipError_t gemm_go_g(const uint16_t* x, int64_t m, int64_t k, const uint8_t* packed,
                            const void* scales, const void* zeros, int64_t n, int g, void* y,
                            void* ws, size_t ws_bytes, hipStream_t st) {
  if (g % 64 == 0) return gemm_go<TS, TY, true>(x, m, k, packed, scales, zeros, n, g, y, ws, ws_bytes, st);
  return gemm_go<TS, TY, false>(x, m, k, packed, scales, zeros, n, g, y, ws, ws_bytes, st);
}

// ---------------------------------------------------------------------------
// Scratch for callers that cannot allocate (w4a16_matmul_noalloc): room for
// the split-K partials of any shape (the plan never asks for more than
// kSplitKMaxBytes).  Each device holds its own copy from module load until
// the process ends; every call on a device shares it, so calls that overlap
// on one device race.  Nothing in it must start at zero: each split writes
// every partial it covers before the reduction reads it.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kSplitKMaxBytes];

// Device address of `scratch` on the current device, looked up once per
// device with hipGetSymbolAddress (the array's name in host code is only a
// stand-in, not a device address).  Devices past 63 look it up every call.
static std::atomic<void*> g_scratch_ptr[64];

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64) {
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p != nullptr) {
      *out = p;
      return hipSuccess;
    }
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (p == nullptr) return hipErrorInvalidSymbol;
  if (dev >= 0 && dev < 64) g_scratch_ptr[dev].store(p, std::memory_order_release);
  *out = p;
  return hipSuccess;
}

hipError_t launch_w4a16_gemm(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                             const void* scales, const void* zeros, int sz_dtype, int64_t n,
                             int g, void* y, int y_dtype, void* ws, size_t ws_bytes, hipStream_t st) {
  const uint16_t* xb = (const uint16_t*)x;
  if (sz_dtype == W4_F16) {
    if (y_dtype == W4_F32)
      return gemm_go_g<_Float16, float>(xb, m, k, packed, scales, zeros, n, g, y, ws, ws_bytes, st);
    return gemm_go_g<_Float16, __bf16>(xb, m, k, packed, scales, zeros, n, g, y, ws, ws_bytes, st);
  }
  if (y_dtype == W4_F32) return gemm_go_g<float, float>(xb, m, k, packed, scales, zeros, n, g, y, ws, ws_bytes, st);
  return gemm_go_g<float, __bf16>(xb, m, k, packed, scales, zeros, n, g, y, ws, ws_bytes, st);
}

}  // namespace w4
