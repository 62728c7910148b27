// Decode-time fused dequantize-matmul for 1 <= M <= 64 bf16 tokens per
// launch (up to 128 in launches of 64) and groups that are multiples of 128
// columns, any K.
// HBM-bound: the kernel exists to stream the packed codes at full bandwidth
// with as little vector-ALU work per code as possible.
//
// Math.  For a 128-column block b of weight row n (one scale s and
// zero-point zp) and token m:
//   sum_k x[m,k] (q[n,k] - zp) s = s * ( sum_k x[m,k] (128 + q[n,k])
//                                        - (128 + zp) * sum_k x[m,k] )
// ("From Scratch: Building a GPTQ INT4 Quantizer in Pure Python", Step 4,
// inside the product of "Building a From-Scratch Group-Wise INT4
// Quantization Layer for LLaMA Weights", Step 2).  128 + q is an exact
// bfloat16 whose low mantissa bits are the code: a byte permute and one
// and-or turn two nibbles into an operand pair, and v_mfma_f32_16x16x32_bf16
// does the multiply-adds (activations as the A operand, 16 token rows; codes
// as B, 16 weight rows).  The block sums of x come from the same MFMA
// against ones, once per wave.
//
// Work layout.  A workgroup owns 16 * RB weight rows over all of K and has
// one wave per 512-column slice of K.  Each wave keeps the activations of
// its slice in registers for the whole kernel and streams the codes of its
// slice for all 16 * RB rows.  In the MFMA operands lane l serves weight row
// l mod 16 and the 32-column quarter l div 16 of each 128-column block; the
// codes are loaded instead as 256-byte runs of one row per 16 lanes (HBM
// serves long runs better) and regrouped through the wave's own 4 KB of
// LDS.  All loads of a wave are issued before any arithmetic and there is
// no barrier until the waves add their partial sums through LDS at the end,
// so each wave computes as soon as its own data arrives.
// When K is not nw whole slices for at most 16 waves (8 with several token
// blocks) -- the Llama-7B down projection, K = 11008, is one case -- a
// workgroup owns 16 rows and up to 8 waves, and each wave loops over an
// equal share of the slices, the last of which may be partial.
#include <type_traits>

#include "w4_common.h"
#include "w4_internal.h"

namespace w4 {

namespace {

#ifndef W4_GEMV_RB
#define W4_GEMV_RB 2
#endif
constexpr int kSlice = 512;  // columns of K per wave
constexpr int kBlocks = kSlice / 128;

// Codes 2v, 2v+1 of a packed 8-code word as a bf16 pair (128 + q each).
__device__ __forceinline__ uint32_t pair_of(uint32_t p, uint32_t p4, uint32_t v, const NibConst& nk) {
  // byte v of p holds codes 2v (low nibble) and 2v+1; byte v of p >> 4 holds
  // code 2v+1 in its low nibble.  Bytes 1 and 3 of the permute are zero.
  const uint32_t sel = v | 0x0c00u | ((4u + v) << 16) | 0x0c000000u;
  return nk(__builtin_amdgcn_perm(p4, p, sel));
}

__device__ __forceinline__ bf16x8 word_to_bf16(uint32_t p, const NibConst& nk) {
  const uint32_t p4 = p >> 4;
  const u32x4 r = {pair_of(p, p4, 0, nk), pair_of(p, p4, 1, nk), pair_of(p, p4, 2, nk),
                   pair_of(p, p4, 3, nk)};
  return __builtin_bit_cast(bf16x8, r);
}

template <typename TS> struct GV;
template <> struct GV<_Float16> {
  typedef uint16_t T;
  typedef u32x2 V4;  // four consecutive scales
  __device__ static float f(T v) { return (float)__builtin_bit_cast(_Float16, v); }
  __device__ static T at(const V4& v, int i) {
    return (T)(((i < 2 ? v.x : v.y) >> (16 * (i & 1))) & 0xffffu);
  }
};
template <> struct GV<float> {
  typedef uint32_t T;
  typedef u32x4 V4;
  __device__ static float f(T v) { return __uint_as_float(v); }
  __device__ static T at(const V4& v, int i) { return v[i]; }
};

template <typename TY>
__device__ __forceinline__ void put1(void* y, int64_t i, float v) {
  if constexpr (sizeof(TY) == 4) {
    ((float*)y)[i] = v;
  } else {
    ((uint16_t*)y)[i] = (uint16_t)f32_to_bf16_bits(v);
  }
}

}  // namespace

// MT: token blocks of 16 (1..4), or 0 for exactly one token (then only
// accumulator element 0 is live).  The token blocks are processed one after
// the other with the wave's codes held in registers, so the codes are read
// from memory once whatever M is.
// G128: group size 128 (the four scales of a slice are contiguous).
template <typename TS, typename TY, int RB, int MT, bool G128, bool SL>
__global__ __launch_bounds__((MT >= 2 || SL) ? 512 : 1024) void k_w4a16_gemv(
    const uint16_t* __restrict__ x, int M, int64_t K, const uint8_t* __restrict__ packed,
    const void* __restrict__ scales, const void* __restrict__ zeros, int64_t N, int g, int ng,
    void* __restrict__ y) {
  typedef typename GV<TS>::T R;
  typedef typename GV<TS>::V4 V4;
  constexpr bool M1 = MT == 0;
  constexpr int T = M1 ? 1 : MT;
  // [waves][RB][16 T tokens][16 rows] partial sums; before them, 4 KB per wave
  // for regrouping activations
  extern __shared__ __attribute__((aligned(16))) float part[];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int l16 = lane & 15, h = lane >> 4;
  const int64_t r0 = (int64_t)blockIdx.x * (16 * RB);
  // SL: K is not nw whole slices, so the waves loop over slices w, w + nw,
  // ... and the last slice may hold fewer than kBlocks blocks (nb): its
  // missing blocks reuse the last block's addresses and contribute nothing
  // (zero scale).  Otherwise wave w takes exactly slice w.
  int64_t k0 = (int64_t)kSlice * w;
  int nb = kBlocks;
  auto blk = [&](int i) { return SL ? (i < nb ? i : nb - 1) : i; };

  // activations of token block tb: the MFMA operand of lane (l16, h) is token
  // 16 tb + l16 (tokens past M repeat the last one and are never stored),
  // columns k0 + 128 i + 32 h + 8 j .. + 7.
  u32x4 xf[kBlocks][4];
  // Several tokens: the block's 16 x 128 activations are loaded with 16
  // consecutive lanes on one token's 256 contiguous bytes (xr), then regrouped
  // into operand order through the wave's own 4 KB of LDS, one 128-column
  // block at a time.  LDS holds token t's 16-byte chunk c at slot c ^ t, so
  // the stores and the operand reads (16 tokens, one chunk) are free of bank
  // conflicts.  LDS operations of a wave complete in order, so the region is
  // reused block after block without a wait.
  u32x4 xr[kBlocks][4];
  auto xload = [&](int tb) {
    if constexpr (M1) {
      const u32x4* xp = (const u32x4*)(x + k0 + 32 * h);
#pragma unroll
      for (int i = 0; i < kBlocks; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) xf[i][j] = xp[16 * blk(i) + j];
    } else {
      // a uniform base (this slice of x) plus a 32-bit lane offset: token
      // tok's row starts tok * 2K bytes in, computed as (tok * K/128) << 8
      // with full-rate 24-bit multiplies (tok < 64, K/128 <= 2^16)
      const char* xb = (const char*)(x + k0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        int tok = 16 * tb + 4 * q + h;
        tok = tok < M ? tok : M - 1;
        const uint32_t xo = (__umul24((uint32_t)tok, (uint32_t)(K / 128)) << 8) + 16u * (uint32_t)l16;
#pragma unroll
        for (int i = 0; i < kBlocks; ++i) xr[i][q] = *(const u32x4*)(xb + xo + 256u * (uint32_t)blk(i));
      }
    }
  };
  auto xstage = [&]() {
    if constexpr (!M1) {
      u32x4* st = (u32x4*)part + 256 * w;
#pragma unroll
      for (int i = 0; i < kBlocks; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int t = 4 * q + h;
          st[16 * t + (l16 ^ t)] = xr[i][q];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) xf[i][j] = st[16 * l16 + ((4 * h + j) ^ l16)];
      }
    }
  };

  // Rows of the workgroup that exist (rows past N repeat the last one and
  // are never stored).  Every weight-side load below is a uniform base at
  // row r0 plus a 32-bit lane offset of at most 16 RB rows, formed with
  // full-rate 24-bit multiplies (row < 64, K/2 <= 2^22, ng <= 2^16).
  const int nvr = (int)(N - r0 < 16 * RB ? N - r0 : 16 * RB);
  uint32_t srow[RB];  // byte offset of the lane's scale row
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int rr = 16 * rb + l16 < nvr ? 16 * rb + l16 : nvr - 1;
    srow[rb] = __umul24((uint32_t)rr, (uint32_t)ng * (uint32_t)sizeof(R));
  }
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
  const NibConst nk = NibConst::make();
  // lane holds tokens 16 tb + 4h + r (r = 0..3) of weight row l16
  f32x4 acc[RB][T];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int tb = 0; tb < T; ++tb) acc[rb][tb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // one slice: loads, then the products of every token block into acc
  auto slice = [&]() {
    // ---- every load of the wave, in the order the arithmetic needs them ----
    xload(0);
    // scales and zero-points of the lane's row for the slice's four blocks
    R sv[RB][kBlocks], zv[RB][kBlocks];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (G128 && (!SL || (ng % kBlocks == 0 && nb == kBlocks))) {  // 4 aligned, in-range scales
        const char* sb = (const char*)((const R*)scales + r0 * ng + k0 / 128);
        const char* zb = (const char*)((const R*)zeros + r0 * ng + k0 / 128);
        const V4 s4 = *(const V4*)(sb + srow[rb]);
        const V4 z4 = *(const V4*)(zb + srow[rb]);
#pragma unroll
        for (int i = 0; i < kBlocks; ++i) {
          sv[rb][i] = GV<TS>::at(s4, i);
          zv[rb][i] = GV<TS>::at(z4, i);
        }
      } else {
#pragma unroll
        for (int i = 0; i < kBlocks; ++i) {
          const int gi = (int)((k0 + 128 * blk(i)) / g);
          const char* sb = (const char*)((const R*)scales + r0 * ng + gi);
          const char* zb = (const char*)((const R*)zeros + r0 * ng + gi);
          sv[rb][i] = *(const R*)(sb + srow[rb]);
          zv[rb][i] = *(const R*)(zb + srow[rb]);
        }
      }
    }
    // packed codes, in 256-byte row runs: row 16 rb + 4 j + h of the
    // workgroup, 16-byte chunk l16 of the slice's run (chunks past the
    // slice's blocks repeat its last chunk)
    u32x4 cr[RB][4];
    {
      const char* cb = (const char*)(packed + r0 * (K / 2) + k0 / 2);
      const uint32_t c16 = 16u * (uint32_t)(l16 < 4 * nb ? l16 : 4 * nb - 1);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rr = 16 * rb + 4 * j + h < nvr ? 16 * rb + 4 * j + h : nvr - 1;
          const uint32_t co = __umul24((uint32_t)rr, (uint32_t)(K / 2)) + c16;
          cr[rb][j] = __builtin_nontemporal_load((const u32x4*)(cb + co));
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // regroup through the wave's LDS region into operand order: lane (l16,
    // h) takes row l16, chunk 4 i + h of block i (row t's chunk c at slot
    // c ^ t, free of bank conflicts; LDS operations of a wave complete in
    // order, so the region is reused row block after row block and then by
    // the activations)
    u32x4 wq[RB][kBlocks];
    {
      u32x4* st = (u32x4*)part + 256 * w;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int t = 4 * j + h;
          st[16 * t + (l16 ^ t)] = cr[rb][j];
        }
#pragma unroll
        for (int i = 0; i < kBlocks; ++i) wq[rb][i] = st[16 * l16 + ((4 * blk(i) + h) ^ l16)];
      }
    }

#pragma unroll
    for (int tb = 0; tb < T; ++tb) {
      if (tb > 0) xload(tb);
      xstage();
      // block sums of x for every token (MFMA against ones)
      f32x4 xs[kBlocks];
#pragma unroll
      for (int i = 0; i < kBlocks; ++i) {
        xs[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          xs[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xf[i][j]), ones, xs[i], 0, 0, 0);
      }
      // row blocks: codes -> bf16 operands, MFMAs, scale and zero-point
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int i = 0; i < kBlocks; ++i) {
          const uint32_t wd[4] = {wq[rb][i].x, wq[rb][i].y, wq[rb][i].z, wq[rb][i].w};
          f32x4 d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int j = 0; j < 4; ++j)
            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xf[i][j]),
                                                        word_to_bf16(wd[j], nk), d, 0, 0, 0);
          const float s = (!SL || i < nb) ? GV<TS>::f(sv[rb][i]) : 0.0f;
          const float nsz = -s * (128.0f + GV<TS>::f(zv[rb][i]));
          if constexpr (M1) {
            acc[rb][tb][0] = fmaf(s, d[0], fmaf(nsz, xs[i][0], acc[rb][tb][0]));
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[rb][tb][r] = fmaf(s, d[r], fmaf(nsz, xs[i][r], acc[rb][tb][r]));
          }
        }
      }
    }
  };
  if constexpr (SL) {
    const int nblk = (int)(K / 128);
    const int nsl = (nblk + kBlocks - 1) / kBlocks;
    for (int sl = w; sl < nsl; sl += nw) {
      k0 = (int64_t)kSlice * sl;
      nb = nblk - kBlocks * sl < kBlocks ? nblk - kBlocks * sl : kBlocks;
      slice();
    }
  } else {
    slice();
  }

  // ---- partial sums of the waves' K slices -> LDS -> y --------------------
  __syncthreads();  // every wave is done with its regrouping region
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float* p = part + (w * RB + rb) * (256 * T);
    if constexpr (M1) {
      if (h == 0) p[l16] = acc[rb][0][0];
    } else {
#pragma unroll
      for (int tb = 0; tb < T; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) p[(16 * tb + 4 * h + r) * 16 + l16] = acc[rb][tb][r];
    }
  }
  __syncthreads();
  const int tid = threadIdx.x;
  const int mm = M1 ? 1 : M;
  const int outs = RB * 16 * mm;
  for (int o = tid; o < outs; o += blockDim.x) {
    const int rb = o / (16 * mm);
    const int rem = o - rb * 16 * mm;
    const int t = rem >> 4, row = rem & 15;
    float s = 0.0f;
    for (int v = 0; v < nw; ++v) s += part[(v * RB + rb) * (256 * T) + t * 16 + row];
    const int64_t n = r0 + 16 * rb + row;
    if (n < N) put1<TY>(y, (int64_t)t * N + n, s);
  }
}

bool gemv_mfma_fits(int64_t m, int64_t k, int g) {
  (void)k;  // any K: K % g == 0, so K % 128 == 0
  return g % 128 == 0 && m >= 1 && m <= 128;
}

// Waves per workgroup of the slice-loop form: at most 8, each taking the
// same number of slices of K.
static int gemv_waves(int64_t k) {
  const int nsl = (int)((k / 128 + kBlocks - 1) / kBlocks);
  const int per = (nsl + 7) / 8;
  return (nsl + per - 1) / per;
}
// One whole slice per wave: the form without the slice loop.
static bool gemv_one_slice(int64_t k, int mt) {
  return k % kSlice == 0 && k / kSlice <= (mt >= 2 ? 8 : 16);
}

template <typename TS, typename TY, int MT, bool G128>
static void gemv_go(const uint16_t* x, int64_t m, int64_t k, const uint8_t* packed,
                    const void* scales, const void* zeros, int64_t n, int g, void* y,
                    hipStream_t st) {
  constexpr int T = MT == 0 ? 1 : MT;
  const size_t stage_per_wave = 4096;  // code and activation regrouping
  if (gemv_one_slice(k, MT)) {
    // W4_GEMV_RB row blocks per workgroup while that still leaves at least
    // one workgroup per CU (256), else one: on [4096,4096] one block is
    // 15-20% faster at every M, on [11008,4096] two are faster at M >= 32.
    const int nw = (int)(k / kSlice);
    auto go = [&](auto rbc) {
      constexpr int RB = decltype(rbc)::value;
      const dim3 grid((unsigned)((n + 16 * RB - 1) / (16 * RB)));
      const size_t part = (size_t)nw * RB * 256 * T * sizeof(float), stage = nw * stage_per_wave;
      k_w4a16_gemv<TS, TY, RB, MT, G128, false><<<grid, 64 * nw, part > stage ? part : stage, st>>>(
          x, (int)m, k, packed, scales, zeros, n, g, (int)(k / g), y);
    };
    if (n >= (int64_t)16 * W4_GEMV_RB * 256) go(std::integral_constant<int, W4_GEMV_RB>{});
    else go(std::integral_constant<int, 1>{});
  } else {
    // slice loop: one row block per workgroup (more workgroups, fewer
    // registers per wave)
    constexpr int RB = 1;
    const int nw = gemv_waves(k);
    const dim3 grid((unsigned)((n + 16 * RB - 1) / (16 * RB)));
    const size_t part = (size_t)nw * RB * 256 * T * sizeof(float), stage = nw * stage_per_wave;
    k_w4a16_gemv<TS, TY, RB, MT, G128, true><<<grid, 64 * nw, part > stage ? part : stage, st>>>(
        x, (int)m, k, packed, scales, zeros, n, g, (int)(k / g), y);
  }
}

template <typename TS, typename TY, bool G128>
static void gemv_pick(const uint16_t* x, int64_t m, int64_t k, const uint8_t* packed,
                      const void* scales, const void* zeros, int64_t n, int g, void* y,
                      hipStream_t st) {
  if (m == 1) gemv_go<TS, TY, 0, G128>(x, m, k, packed, scales, zeros, n, g, y, st);
  else if (m <= 16) gemv_go<TS, TY, 1, G128>(x, m, k, packed, scales, zeros, n, g, y, st);
  else if (m <= 32) gemv_go<TS, TY, 2, G128>(x, m, k, packed, scales, zeros, n, g, y, st);
  else if (m <= 48) gemv_go<TS, TY, 3, G128>(x, m, k, packed, scales, zeros, n, g, y, st);
  else if (!gemv_one_slice(k, 4)) {
    // The slice-loop form with four token blocks runs out of registers; two
    // launches of up to 32 tokens each are faster.
    gemv_go<TS, TY, 2, G128>(x, 32, k, packed, scales, zeros, n, g, y, st);
    gemv_go<TS, TY, 2, G128>(x + 32 * k, m - 32, k, packed, scales, zeros, n, g,
                             (char*)y + 32 * n * (int64_t)sizeof(TY), st);
  } else gemv_go<TS, TY, 4, G128>(x, m, k, packed, scales, zeros, n, g, y, st);
}

// More than 64 tokens: launches of up to 64 tokens each, every one reading
// the codes again.  Up to 128 tokens this beats the prefill GEMM, whose
// 256 x 128 tiles then cover few CUs (N / 128 workgroups).
template <typename TS, typename TY>
static void gemv_pick(const uint16_t* x, int64_t m, int64_t k, const uint8_t* packed,
                      const void* scales, const void* zeros, int64_t n, int g, void* y,
                      hipStream_t st) {
  for (int64_t t0 = 0; t0 < m; t0 += 64) {
    const int64_t mc = m - t0 < 64 ? m - t0 : 64;
    const uint16_t* xc = x + t0 * k;
    void* yc = (char*)y + t0 * n * (int64_t)sizeof(TY);
    if (g == 128) gemv_pick<TS, TY, true>(xc, mc, k, packed, scales, zeros, n, g, yc, st);
    else gemv_pick<TS, TY, false>(xc, mc, k, packed, scales, zeros, n, g, yc, st);
  }
}

hipError_t launch_w4a16_gemv(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                             const void* scales, const void* zeros, int sz_dtype, int64_t n,
                             int g, void* y, int y_dtype, hipStream_t st) {
  const uint16_t* xb = (const uint16_t*)x;
  if (sz_dtype == W4_F16) {
    if (y_dtype == W4_F32) gemv_pick<_Float16, float>(xb, m, k, packed, scales, zeros, n, g, y, st);
    else gemv_pick<_Float16, __bf16>(xb, m, k, packed, scales, zeros, n, g, y, st);
  } else {
    if (y_dtype == W4_F32) gemv_pick<float, float>(xb, m, k, packed, scales, zeros, n, g, y, st);
    else gemv_pick<float, __bf16>(xb, m, k, packed, scales, zeros, n, g, y, st);
  }
  return hipGetLastError();
}

}  // namespace w4
