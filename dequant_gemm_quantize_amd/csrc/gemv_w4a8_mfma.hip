// W4A8 GEMV for a few INT8 tokens (1 <= M <= 16), any K, groups that are
// multiples of 128 columns, on the int8 MFMA units.  HBM-bound: the packed
// codes are streamed once.
//
// Math ("Hands-on Build Guide: Group-wise INT4 Weight-only Quantization with
// Per-channel Scales", Step 5):
//   y[m, n] = s_a[m] * sum_g s[n, g] * sum_{k in g} xq[m, k] (q[n, k] - zp[n, g]).
// Each 128-column block lies inside one group.  Its codes become the exact
// int8 values q - zp (the same byte arithmetic as the W4A8 GEMM), and two
// v_mfma_i32_16x16x64_i8 (tokens as the A rows, weight rows as the B
// columns) give the exact int32 block sums, which are scaled by s[n, g] into
// fp32 accumulators; the token scale is applied once at the end.
//
// Work layout (as the bf16 MFMA GEMV): a workgroup owns 16 RB weight rows
// (RB = 1 or 2) and up to 8 waves; each wave loops over an equal share of the 512-column
// slices of K (the last slice may hold fewer than four blocks).  Inside a
// block, lane (r, q) holds weight row r and token r in the two operands and
// the 32 columns 32q .. 32q + 31, 16 per MFMA: one 16-byte code load and two
// 16-byte activation loads per block.  The waves' partial sums meet in LDS at
// the end.
#include <type_traits>

#include "w4_common.h"
#include "w4_internal.h"

namespace w4 {

namespace {

#ifndef W4_W8G_SLICE
#define W4_W8G_SLICE 4
#endif
constexpr int kSliceB = W4_W8G_SLICE;  // 128-column blocks per slice

template <typename TS> struct GA;
template <> struct GA<_Float16> {
  typedef uint16_t T;
  __device__ static float f(T v) { return (float)__builtin_bit_cast(_Float16, v); }
};
template <> struct GA<float> {
  typedef uint32_t T;
  __device__ static float f(T v) { return __uint_as_float(v); }
};

// 8 codes of a packed word -> 8 int8 values q - zp in column order, given
// c = 0x80808080 - zp * 0x01010101: per byte q + 128 - zp lies in [113, 143],
// so the add has no carries, and flipping bit 7 gives the two's complement
// byte of q - zp.
__device__ __forceinline__ u32x2 centre8v(uint32_t p, uint32_t c) {
  const uint32_t lo = (p & 0x0f0f0f0fu) + c;         // codes 0, 2, 4, 6
  const uint32_t hi = ((p >> 4) & 0x0f0f0f0fu) + c;  // codes 1, 3, 5, 7
  u32x2 r;
  r.x = __builtin_amdgcn_perm(hi, lo, 0x05010400u) ^ 0x80808080u;  // 0 1 2 3
  r.y = __builtin_amdgcn_perm(hi, lo, 0x07030602u) ^ 0x80808080u;  // 4 5 6 7
  return r;
}

template <typename TY>
__device__ __forceinline__ void put8m(void* y, int64_t i, float v) {
  if constexpr (sizeof(TY) == 4) {
    ((float*)y)[i] = v;
  } else {
    ((uint16_t*)y)[i] = (uint16_t)f32_to_bf16_bits(v);
  }
}

}  // namespace

template <typename TS, typename TY, int RB>
__global__ __launch_bounds__(512) void k_w4a8_gemv_mfma(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, int M, int64_t K,
    const uint8_t* __restrict__ packed, const void* __restrict__ scales,
    const void* __restrict__ zeros, int64_t N, int g, void* __restrict__ y) {
  typedef typename GA<TS>::T R;
  // LDS: per wave 4 KB for regrouping the codes of a slice, then
  // [waves][RB][16 tokens][16 rows] partial sums
  extern __shared__ __attribute__((aligned(16))) unsigned char lds8[];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * (16 * RB);
  const int64_t ng = K / g;
  const int nblk = (int)(K / 128);
  const int nsl = (nblk + kSliceB - 1) / kSliceB;
  constexpr int CPR = 4 * kSliceB;  // 16-byte code chunks per row and slice
  // per wave: 16 tokens x the slice's 512 bytes of activations (8 KB), reused
  // for the codes' regrouping (4 KB)
  constexpr int XCH = 2 * CPR;          // 16-byte activation chunks per token and slice
  constexpr int XPL = XCH / 16;         // of them per lane and token group
  constexpr int XSLOTS = 16 * XCH;      // 16-byte slots: 16 tokens x XCH chunks
  u32x4* stg = (u32x4*)lds8 + XSLOTS * w;
  float* part8 = (float*)(lds8 + (size_t)nw * 16 * XSLOTS);

  // Code loads: 16 consecutive lanes read one row's 256 contiguous bytes of
  // the slice (4 rows per instruction); the slice is then regrouped through
  // the wave's 4 KB of LDS into operand order (lane (r, q) takes row r,
  // bytes 64 b + 16 q of block b).  Row t's chunk c sits at slot c ^ t, so
  // stores and operand reads are free of bank conflicts, and LDS operations
  // of a wave complete in order, so the region is reused row block after
  // row block and slice after slice.  The RB row blocks of the workgroup
  // share the activation registers, which are the larger read at 16 tokens.
  const uint8_t* crow[RB][4];
  const R* srow[RB];
  const R* zrow[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int64_t rj = n0 + 16 * rb + 4 * j + q;
      rj = rj < N ? rj : N - 1;
      crow[rb][j] = packed + rj * (K / 2);
    }
    int64_t row = n0 + 16 * rb + r16;
    row = row < N ? row : N - 1;
    srow[rb] = (const R*)scales + row * ng;
    zrow[rb] = (const R*)zeros + row * ng;
  }
  // activation loads: 16 consecutive lanes read 256 contiguous bytes of one
  // token (token 4u + q, chunks r16 + 16 s of the slice's run), regrouped
  // through LDS into operand order (lane (r, q) of half j of block i takes
  // token r, chunk 8 i + 2 q + j); token t's chunk c at slot XCH t + (c ^ t),
  // free of bank conflicts both ways
  const u32x4* xtok[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    int t = 4 * u + q;
    t = t < M ? t : M - 1;  // tokens past M repeat the last one
    xtok[u] = (const u32x4*)(xq + (int64_t)t * K);
  }

  f32x4 acc[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int sl = w; sl < nsl; sl += nw) {
    const int b0 = kSliceB * sl;
    const int nb = nblk - b0 < kSliceB ? nblk - b0 : kSliceB;
    // ---- loads: codes (coalesced), activations, scales / zero-points ------
    u32x4 cr[RB][4][CPR / 16], xa[kSliceB][2];
    R sv[RB][kSliceB], zv[RB][kSliceB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int h = 0; h < CPR / 16; ++h) {
          const int c = r16 + 16 * h;
          const int cc = c < 4 * nb ? c : 4 * nb - 1;  // chunk of the slice's run
          cr[rb][j][h] = __builtin_nontemporal_load((const u32x4*)(crow[rb][j] + (int64_t)b0 * 64) + cc);
        }
    u32x4 xr[4][XPL];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int s2 = 0; s2 < XPL; ++s2) {
        const int c = r16 + 16 * s2;
        const int cc = c < 8 * nb ? c : 8 * nb - 1;  // chunk of the slice's run
        xr[u][s2] = xtok[u][8 * b0 + cc];
      }
#pragma unroll
    for (int i = 0; i < kSliceB; ++i) {
      const int b = b0 + (i < nb ? i : nb - 1);  // missing blocks reuse the last
      const int64_t gi = (int64_t)b * 128 / g;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        sv[rb][i] = srow[rb][gi];
        zv[rb][i] = zrow[rb][gi];
      }
    }
    // ---- regroup the activations into operand order ------------------------
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int s2 = 0; s2 < XPL; ++s2) {
        const int t = 4 * u + q, c = r16 + 16 * s2;
        stg[XCH * t + (c ^ t)] = xr[u][s2];
      }
#pragma unroll
    for (int i = 0; i < kSliceB; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = 8 * i + 2 * q + j;  // the columns of the codes' half j (bw0 / bw1)
        xa[i][j] = stg[XCH * r16 + (c ^ r16)];
      }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      // ---- regroup the codes: row 4j + q, chunk r16 -> operand order -------
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 4 * j + q;
#pragma unroll
        for (int h = 0; h < CPR / 16; ++h) stg[CPR * t + ((r16 + 16 * h) ^ t)] = cr[rb][j][h];
      }
      u32x4 wq[kSliceB];
#pragma unroll
      for (int i = 0; i < kSliceB; ++i) wq[i] = stg[CPR * r16 + ((4 * i + q) ^ r16)];
      // ---- per block: int8 (q - zp), two MFMAs, scale into acc -----------
#pragma unroll
      for (int i = 0; i < kSliceB; ++i) {
        const uint32_t c = 0x80808080u - (uint32_t)GA<TS>::f(zv[rb][i]) * 0x01010101u;
        const u32x2 e0 = centre8v(wq[i].x, c), e1 = centre8v(wq[i].y, c);
        const u32x2 e2 = centre8v(wq[i].z, c), e3 = centre8v(wq[i].w, c);
        const i32x4 bw0 = __builtin_bit_cast(i32x4, u32x4{e0.x, e0.y, e1.x, e1.y});
        const i32x4 bw1 = __builtin_bit_cast(i32x4, u32x4{e2.x, e2.y, e3.x, e3.y});
        i32x4 d = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, xa[i][0]), bw0,
                                                       i32x4{0, 0, 0, 0}, 0, 0, 0);
        d = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, xa[i][1]), bw1, d, 0, 0, 0);
        const float s = i < nb ? GA<TS>::f(sv[rb][i]) : 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[rb][r] = fmaf(s, (float)d[r], acc[rb][r]);
      }
    }
  }

  // ---- lane holds tokens 4q + r of weight row 16 rb + r16; waves -> LDS -> y
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 4; ++r) part8[((w * RB + rb) * 16 + 4 * q + r) * 16 + r16] = acc[rb][r];
  __syncthreads();
  for (int o = threadIdx.x; o < RB * 16 * M; o += blockDim.x) {
    const int rb = o / (16 * M);
    const int rem = o - rb * 16 * M;
    const int t = rem >> 4, rr = rem & 15;
    float sum = 0.0f;
    for (int v = 0; v < nw; ++v) sum += part8[((v * RB + rb) * 16 + t) * 16 + rr];
    const int64_t n = n0 + 16 * rb + rr;
    if (n < N) put8m<TY>(y, (int64_t)t * N + n, xs[t] * sum);
  }
}

bool w4a8_gemv_mfma_fits(int64_t m, int64_t k, int g) {
  (void)k;  // any K: K % g == 0, so K % 128 == 0
  return m >= 1 && m <= 16 && g % 128 == 0;
}

template <typename TS, typename TY>
static void w4a8_mfma_go(const int8_t* xq, const float* xs, int64_t m, int64_t k,
                         const uint8_t* packed, const void* scales, const void* zeros, int64_t n,
                         int g, void* y, hipStream_t st) {
  const int nsl = (int)((k / 128 + kSliceB - 1) / kSliceB);
  const int per = (nsl + 7) / 8;
  const int nw = (nsl + per - 1) / per;  // at most 8 waves, equal shares of slices
  auto go = [&](auto rbc) {
    constexpr int RB = decltype(rbc)::value;
    const dim3 grid((unsigned)((n + 16 * RB - 1) / (16 * RB)));
    const size_t lds = (size_t)nw * (16 * 16 * 2 * 4 * kSliceB + RB * 256 * sizeof(float));  // 16 XSLOTS bytes
    k_w4a8_gemv_mfma<TS, TY, RB><<<grid, 64 * nw, lds, st>>>(xq, xs, (int)m, k, packed, scales, zeros,
                                                             n, g, y);
  };
  // Two row blocks per workgroup when each wave loops over many slices (long
  // K) and a workgroup per CU remains: on [8192,28672] 61 -> 52 us at 16
  // tokens; on [28672,8192] (two slices per wave) one block is 10% faster.
  if (k >= 16384 && n >= 16 * 2 * 256) go(std::integral_constant<int, 2>{});
  else go(std::integral_constant<int, 1>{});
}

hipError_t launch_w4a8_gemv_mfma(const int8_t* xq, const float* xs, int64_t m, int64_t k,
                                 const uint8_t* packed, const void* scales, const void* zeros,
                                 int sz_dtype, int64_t n, int g, void* y, int y_dtype,
                                 hipStream_t st) {
  if (sz_dtype == W4_F16) {
    if (y_dtype == W4_F32) w4a8_mfma_go<_Float16, float>(xq, xs, m, k, packed, scales, zeros, n, g, y, st);
    else w4a8_mfma_go<_Float16, __bf16>(xq, xs, m, k, packed, scales, zeros, n, g, y, st);
  } else {
    if (y_dtype == W4_F32) w4a8_mfma_go<float, float>(xq, xs, m, k, packed, scales, zeros, n, g, y, st);
    else w4a8_mfma_go<float, __bf16>(xq, xs, m, k, packed, scales, zeros, n, g, y, st);
  }
  return hipGetLastError();
}

}  // namespace w4
