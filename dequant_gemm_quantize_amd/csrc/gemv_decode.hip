// Decode-time fused dequantize-matmul for 2 <= M <= 4 tokens (bf16 x) whose
// activations fit in LDS, groups that are multiples of 128 columns, at the
// shapes the 4x4x4 matrix-core GEMV does not take (K other than 4096).
// HBM-bound: the kernels exist to stream the packed codes at full bandwidth.
//
// Math.  For a 128-column block b of weight row n (inside one group, scale s,
// zero-point zp) and token m:
//   sum_k x[m,k] * (q[n,k] - zp) * s
//     = s * ( sum_k x[m,k] * (128 + q[n,k])  -  (128 + zp) * sum_k x[m,k] )
// ("From Scratch: Building a GPTQ INT4 Quantizer in Pure Python", Step 4,
// inside the product of "Building a From-Scratch Group-Wise INT4 Quantization
// Layer for LLaMA Weights", Step 2).  128 + q is an exact bfloat16 whose low
// mantissa bits are the code, so a nibble becomes an MFMA operand with a
// shift and one and-or per pair of codes.  Both sums run on the bf16 MFMA
// unit (v_mfma_f32_16x16x32_bf16): the first against the codes, the second
// against the constant -(128 + zp) of the row, into the same fp32
// accumulator.  The block result is scaled by s with one FMA per output.
//
// Work layout.  A 256-lane workgroup owns 16 weight rows (one MFMA column
// each) over all of K; its four waves split K into contiguous ranges and add
// their 16x16 partial tiles through LDS at the end.  Lane l serves weight row
// (l mod 16) and k-group (l div 16): per block it loads 16 bytes of packed
// codes (32 consecutive columns).  Each wave stages its activations, scales
// and zero-points in its own LDS region (no workgroup barrier), and packed
// loads for up to 8 blocks are in flight per lane before the first MFMA.
#include "w4_common.h"
#include "w4_internal.h"

namespace w4 {

namespace {

#ifndef W4_DECODE_CHUNK
#define W4_DECODE_CHUNK 8
#endif
constexpr int kRows = 16;                // weight rows per workgroup
constexpr int kChunk = W4_DECODE_CHUNK;  // 128-column blocks whose codes are loaded ahead


template <typename TY>
__device__ __forceinline__ void store_out(void* y, int64_t i, float v) {
  if constexpr (sizeof(TY) == 4) {
    ((float*)y)[i] = v;
  } else {
    ((uint16_t*)y)[i] = (uint16_t)f32_to_bf16_bits(v);
  }
}

}  // namespace

// Raw (unconverted) scale / zero-point element of the storage dtype.
template <typename TS> struct RawSZ;
template <> struct RawSZ<_Float16> {
  typedef uint16_t T;
  __device__ static float scale(T v) { return (float)__builtin_bit_cast(_Float16, v); }
  __device__ static uint32_t zero(T v) { return (uint32_t)(float)__builtin_bit_cast(_Float16, v); }
};
template <> struct RawSZ<float> {
  typedef uint32_t T;
  __device__ static float scale(T v) { return __uint_as_float(v); }
  __device__ static uint32_t zero(T v) { return (uint32_t)__uint_as_float(v); }
};

// ---------------------------------------------------------------------------
// The decode kernel (used when the activations fit the LDS budget of
// 64 KB).  Two details cut registers
// and VALU work:
//  * the block's codes are expanded in the order (0,4), (1,5), (2,6), (3,7)
//    of each 8-code word -- seven instructions per word (shift + and-or) --
//    and the activations are stored in LDS in that same order, so the MFMA
//    still pairs every code with its own activation;
//  * operands are read from LDS just before use (ds_read_b128), so no
//    activation registers are held across blocks.
// ---------------------------------------------------------------------------
#ifndef W4_DECODE_LDS_BYTES
#define W4_DECODE_LDS_BYTES 65536
#endif
constexpr int kDecodeLds = W4_DECODE_LDS_BYTES;

// Codes 0..7 of a word as bf16 pairs (128+q) in the order (0,4),(1,5),(2,6),(3,7).
__device__ __forceinline__ bf16x8 codes_to_bf16_interleaved(uint32_t p) {
  u32x4 r;
  const NibConst nk = NibConst::make();
  r.x = nk(p);
  r.y = nk(p >> 4);
  r.z = nk(p >> 8);
  r.w = nk(p >> 12);
  return __builtin_bit_cast(bf16x8, r);
}

// 8 bf16 activations (x0..x7 as 4 pairs) -> pairs (x0,x4),(x1,x5),(x2,x6),(x3,x7).
__device__ __forceinline__ u32x4 interleave8(u32x4 v) {
  u32x4 r;
  r.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);  // lo(v.x), lo(v.z)
  r.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);  // hi(v.x), hi(v.z)
  r.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
  r.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
  return r;
}

// MFMAs of CH consecutive blocks whose codes are already loaded (wq); block
// i waits only for its own codes (vmcnt retires in order).  Scale and
// zero-point of every block come from the LDS tile.
template <int CH>
__device__ __forceinline__ void decode_math(const u32x4 (&wq)[CH], const u32x4* __restrict__ xl,
                                            const float* __restrict__ s_l,
                                            const uint32_t* __restrict__ zb_l, int c0,
                                            f32x4& acc) {
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const uint32_t zb = zb_l[c0 + i];
    const bf16x8 bz = __builtin_bit_cast(bf16x8, u32x4{zb, zb, zb, zb});
    const uint32_t w4[4] = {wq[i].x, wq[i].y, wq[i].z, wq[i].w};
    f32x4 ga = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, xl[16 * (c0 + i) + t]);
      ga = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, codes_to_bf16_interleaved(w4[t]), ga, 0, 0, 0);
      ga = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bz, ga, 0, 0, 0);
    }
    const float sc = s_l[c0 + i];
    acc.x = fmaf(sc, ga.x, acc.x);
    acc.y = fmaf(sc, ga.y, acc.y);
    acc.z = fmaf(sc, ga.z, acc.z);
    acc.w = fmaf(sc, ga.w, acc.w);
  }
}

template <int CH>
__device__ __forceinline__ void decode_loads(const u32x4* __restrict__ wrow, int c0, u32x4 (&wq)[CH]) {
#pragma unroll
  for (int i = 0; i < CH; ++i) wq[i] = wrow[4 * (c0 + i)];
}

// c0: absolute block (codes in memory); r0: block relative to the wave's
// first block (LDS slices).
template <int CH>
__device__ __forceinline__ void decode_blocks(const u32x4* __restrict__ wrow,
                                              const u32x4* __restrict__ xl,
                                              const float* __restrict__ s_l,
                                              const uint32_t* __restrict__ zb_l, int c0, int r0,
                                              f32x4& acc) {
  u32x4 wq[CH];
  decode_loads<CH>(wrow, c0, wq);
  __builtin_amdgcn_sched_barrier(0);
  decode_math<CH>(wq, xl, s_l, zb_l, r0, acc);
}

// LDS layout of the decode kernel (dynamic shared memory), one private
// region per wave -- staging needs no workgroup barrier:
//   sc[16][nblk]  float   scale of (tile row, block), absolute block index
//   zb[16][nblk]  uint32  bf16 pair -(128 + zp) of (tile row, block)
//   x [M][nw*16]  16-byte groups of the wave's activations, interleaved order
// followed by part[WAVES][64] f32x4 for the final cross-wave sum.  A wave
// fills only the blocks it uses.
__host__ __device__ inline int64_t decode_wave_blocks(int64_t k, int waves) {
  const int64_t nblk = k / 128;
  return (nblk + waves - 1) / waves;  // upper bound of blocks per wave
}
__host__ __device__ inline int64_t decode_wave_bytes(int64_t m, int64_t k, int waves) {
  return 16 * (k / 128) * 8 + m * decode_wave_blocks(k, waves) * 256;
}
size_t decode_lds_bytes(int64_t m, int64_t k, int waves) {
  return (size_t)(waves * decode_wave_bytes(m, k, waves) + waves * 64 * 16);
}

template <typename TS, typename TY, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_w4a16_decode(
    const uint16_t* __restrict__ x, int M, int64_t K, const uint8_t* __restrict__ packed,
    const void* __restrict__ scales, const void* __restrict__ zeros, int64_t N, int g,
    void* __restrict__ y) {
  typedef typename RawSZ<TS>::T R;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int j = lane & 15;
  const int kg = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * kRows;
  const int64_t n = (n0 + j < N) ? (n0 + j) : (N - 1);
  const int nblk = (int)(K / 128);
  const int ng = (int)(K / g);
  const int bpg = g / 128;
  const int b0 = (wave * nblk) / WAVES;
  const int b1 = ((wave + 1) * nblk) / WAVES;
  const int nwb = b1 - b0;                                  // this wave's blocks
  unsigned char* base = lds + (int64_t)wave * decode_wave_bytes(M, K, WAVES);
  float* sc_l = (float*)base;                               // [16][nblk]
  uint32_t* zb_l = (uint32_t*)(base + 16 * nblk * 4);       // [16][nblk]
  // [M][nwb*16]; the region is sized for the largest wave share,
  // decode_wave_blocks(K, WAVES) blocks
  u32x4* xs_l = (u32x4*)(base + 16 * nblk * 8);
  f32x4* part = (f32x4*)(lds + (int64_t)WAVES * decode_wave_bytes(M, K, WAVES));

  const R* sg = (const R*)scales;
  const R* zg = (const R*)zeros;
  const u32x4* xg = (const u32x4*)x;
  const u32x4* wrow = (const u32x4*)(packed + n * (K / 2)) + kg;

  // ---- 1. codes of the first chunk ---------------------------------------
  const bool first_full = nwb >= kChunk;
  u32x4 wq0[kChunk];
  if (first_full) decode_loads<kChunk>(wrow, b0, wq0);
  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. LDS stores of the wave's slices (no workgroup barrier) -----------
  for (int i = lane; i < M * nwb * 16; i += 64) {
    const int m = i / (nwb * 16), c = i - m * (nwb * 16);
    xs_l[i] = interleave8(xg[(int64_t)m * (K / 8) + b0 * 16 + c]);
  }
  for (int e = lane; e < 16 * nwb; e += 64) {
    const int row = e / nwb, b = b0 + (e - row * nwb);
    int64_t ge = (n0 + row < N ? n0 + row : N - 1) * ng + b / bpg;
    sc_l[row * nblk + b] = RawSZ<TS>::scale(sg[ge]);
    zb_l[row * nblk + b] = (0xc300u | RawSZ<TS>::zero(zg[ge])) * 0x00010001u;
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's LDS stores are done
  __builtin_amdgcn_wave_barrier();

  // ---- 3. MFMAs over the wave's blocks (block-relative LDS indices) --------
  const int jx = j < M ? j : 0;  // operand rows m >= M repeat token 0 (never stored)
  const u32x4* xl = xs_l + jx * (nwb * 16) + kg * 4;  // indexed by block relative to b0
  const float* s_l = sc_l + j * nblk + b0;   // indexed by block relative to b0
  const uint32_t* z_l = zb_l + j * nblk + b0;

  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  int c0 = b0;
  if (first_full) {
    decode_math<kChunk>(wq0, xl, s_l, z_l, 0, acc);
    c0 += kChunk;
  }
  for (; c0 + kChunk <= b1; c0 += kChunk) decode_blocks<kChunk>(wrow, xl, s_l, z_l, c0, c0 - b0, acc);
  if (kChunk > 4 && c0 + 4 <= b1) { decode_blocks<4>(wrow, xl, s_l, z_l, c0, c0 - b0, acc); c0 += 4; }
  if (kChunk > 2 && c0 + 2 <= b1) { decode_blocks<2>(wrow, xl, s_l, z_l, c0, c0 - b0, acc); c0 += 2; }
  if (c0 < b1) decode_blocks<1>(wrow, xl, s_l, z_l, c0, c0 - b0, acc);

  // ---- 4. cross-wave sum of the partial tiles, store -----------------------
  part[wave * 64 + lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4 sum = part[lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) {
      const f32x4 o = part[w * 64 + lane];
      sum.x += o.x; sum.y += o.y; sum.z += o.z; sum.w += o.w;
    }
    if (n0 + j < N) {
      const float v[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * kg + r;
        if (m < M) store_out<TY>(y, (int64_t)m * N + n0 + j, v[r]);
      }
    }
  }
}

#ifndef W4_DECODE_WAVES
#define W4_DECODE_WAVES 4
#endif

bool decode_lds_fits(int64_t m, int64_t k) {
  return decode_lds_bytes(m, k, W4_DECODE_WAVES) <= (size_t)kDecodeLds;
}

template <typename TS, typename TY>
static void decode_go(dim3 grid, hipStream_t st, const uint16_t* x, int M, int64_t k,
                      const uint8_t* packed, const void* scales, const void* zeros, int64_t n,
                      int g, void* y) {
  // (one token never gets here: it goes to the dot2 GEMV; two to four
  // tokens at K = 4096 go to the 4x4x4 matrix-core GEMV)
  constexpr int W = W4_DECODE_WAVES;
  const size_t lds = decode_lds_bytes(M, k, W);
  k_w4a16_decode<TS, TY, W><<<grid, 64 * W, lds, st>>>(x, M, k, packed, scales, zeros, n, g, y);
}

hipError_t launch_w4a16_decode(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                               const void* scales, const void* zeros, int sz_dtype, int64_t n,
                               int g, void* y, int y_dtype, hipStream_t st) {
  const dim3 grid((unsigned)((n + kRows - 1) / kRows));
  const uint16_t* xb = (const uint16_t*)x;
  const int M = (int)m;
  if (sz_dtype == W4_F16) {
    if (y_dtype == W4_F32) decode_go<_Float16, float>(grid, st, xb, M, k, packed, scales, zeros, n, g, y);
    else decode_go<_Float16, __bf16>(grid, st, xb, M, k, packed, scales, zeros, n, g, y);
  } else {
    if (y_dtype == W4_F32) decode_go<float, float>(grid, st, xb, M, k, packed, scales, zeros, n, g, y);
    else decode_go<float, __bf16>(grid, st, xb, M, k, packed, scales, zeros, n, g, y);
  }
  return hipGetLastError();
}

}  // namespace w4
