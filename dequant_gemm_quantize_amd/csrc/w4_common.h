// Device-side helpers shared by the libw4 kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
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

// float32 -> bfloat16 bits, round to nearest even (quiet NaN preserved).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
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

}  // namespace w4
