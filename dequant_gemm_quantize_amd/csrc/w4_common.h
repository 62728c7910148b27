// Device-side helpers shared by the libw4 kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---- scalar conversions ----------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}
// Low / high bf16 of a packed pair, widened exactly.
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// float32 -> bfloat16 bits, round to nearest even, NaN quieted with its sign
// and upper payload kept.  The hardware conversion (v_cvt_pk_bf16_f32) gives
// the same bits as the integer form (u + 0x7fff + bit 16) >> 16, with
// (u >> 16) | 0x40 for NaN, on all 2^32 inputs under these kernels' float
// mode (denormals kept); that was checked exhaustively on gfx950.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// float32 -> float16 bits, round to nearest even (hardware conversion).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// Scale / zero-point element access for the two storage dtypes.
template <typename TS> struct ScaleT;
template <> struct ScaleT<float> {
  __device__ static float load(const void* p, int64_t i) { return ((const float*)p)[i]; }
};
template <> struct ScaleT<_Float16> {
  __device__ static float load(const void* p, int64_t i) {
    return (float)((const _Float16*)p)[i];
  }
};

// ---- wave reductions (xor butterflies inside a wave) -------------------------
template <int WIDTH>
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
template <int WIDTH>
__device__ __forceinline__ float group_min(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
  return v;
}
template <int WIDTH>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// ---- non-temporal / plain vector loads -------------------------------------
template <typename T>
__device__ __forceinline__ T ldg_nt(const T* p) {
  return __builtin_nontemporal_load(p);
}

// The two constants of the nibble -> bf16 conversion (q & 0x000f000f) |
// 0x43004300, held in registers.  VOP3 instructions on this target take no
// literal operand, so with plain constants the compiler splits
// v_and_or_b32 into v_and_b32 + v_or_b32.  The empty asm statement emits no
// instruction; it only hides the values from constant folding, and being
// free of side effects it is merged across calls, so the constants are
// materialised once per kernel.  (The and-or itself stays plain C: an
// inline-asm ALU instruction that feeds an MFMA is invisible to the
// compiler's hazard tracking.)
struct NibConst {
  uint32_t mask, magic;
  __device__ static NibConst make() {
    NibConst k{0x000f000fu, 0x43004300u};
    asm("" : "+v"(k.mask), "+v"(k.magic));
    return k;
  }
  __device__ uint32_t operator()(uint32_t p) const { return (p & mask) | magic; }
};

// ---- buffer resources and the MFMA-block store -----------------------------
// Raw buffer resource over `base` (gfx9 word 3: 32-bit data format, no
// swizzle).  Accesses through it take a uniform base, a per-lane VGPR offset
// and a uniform SGPR offset.  Callers keep offsets below 2^31, so the range
// check never triggers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000);
}

// Stores a wave's 64 x 32 NJ block of v_mfma 32x32 accumulators into a
// row-major array of TY (float, or bfloat16 rounded to nearest even) with
// leading dimension ld, for a block that lies wholly inside the array.
// Register r of acc[i][j] holds block row 32 i + 8 (r / 4) + 4 (lane / 32) +
// r % 4, column 32 j + lane % 32; `blk` points at the block's first element.
// With RS, block row t is multiplied by rs[t] first.  blk, rs and ld are the
// same in every lane.  Row offsets are uniform and the lane's offset is fixed, so an element costs its conversion and one
// store, with no bounds test.  Needs 64 * ld * sizeof(TY) < 2^31.
// A pointer that is the same in every lane, moved to scalar registers (the
// compiler cannot always prove it uniform, and a buffer resource in vector
// registers costs a loop per access).
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t u = (uint64_t)p;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  return (T*)(lo | (hi << 32));
}

template <typename TY, int NJ, bool RS>
__device__ __forceinline__ void store_wave_block(void* blk, int64_t ld, int lane,
                                                 const f32x16 (&acc)[2][NJ], const float* rs) {
  const __amdgpu_buffer_rsrc_t yr = buf_rsrc(uniform_ptr(blk));
  const uint32_t l4 = (uint32_t)(lane >> 5);
  const uint32_t vo = (4u * l4 * (uint32_t)ld + (uint32_t)(lane & 31)) * (uint32_t)sizeof(TY);
  // the lane's 32 row factors, all loaded before the first store (the
  // compiler would not move a load across a store through another resource)
  float a[2][16];
  if constexpr (RS) {
    const __amdgpu_buffer_rsrc_t sr = buf_rsrc(uniform_ptr(rs));
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        a[i][r] = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(sr, 16u * l4, 4 * (32 * i + 8 * (r >> 2) + (r & 3)), 0));
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = 32 * i + 8 * (r >> 2) + (r & 3);  // block row, less 4 (lane / 32)
      const uint32_t so = (uint32_t)t * (uint32_t)ld * (uint32_t)sizeof(TY);
      float v[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) v[j] = RS ? acc[i][j][r] * a[i][r] : acc[i][j][r];
      if constexpr (sizeof(TY) == 4) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[j]), yr, vo, so + 128 * j, 0);
      } else {
#pragma unroll
        for (int j = 0; j + 1 < NJ; j += 2) {  // one conversion per pair of columns
          const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){v[j], v[j + 1]}, bf16x2));
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)h, yr, vo, so + 64 * j, 0);
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(h >> 16), yr, vo, so + 64 * j + 64, 0);
        }
        if constexpr (NJ % 2 == 1)
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (__bf16)v[NJ - 1]), yr, vo,
                                                so + 64 * (NJ - 1), 0);
      }
    }
}
}  // namespace w4
