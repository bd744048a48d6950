// Device-side helpers shared by the gfx950 kernels: 16-bit float storage conversions, output
// stores and small vector types.  Everything here is plain HIP for CDNA4 (wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ql {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

// dtype codes (same values as ql_dtype in qlinear.h)
enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

struct BF16 {};  // tag: bfloat16 storage
struct F16 {};   // tag: IEEE binary16 storage

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// Round fp32 to bfloat16, nearest with ties to even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rne = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t nan = (u >> 16) | 0x40u;
  return (u & 0x7fffffffu) > 0x7f800000u ? nan : rne;  // a select, not a branch
}
// Round fp32 to binary16 (the hardware conversion rounds to nearest even).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

template <typename T> __device__ __forceinline__ float param_to_f32(uint32_t bits);
template <> __device__ __forceinline__ float param_to_f32<BF16>(uint32_t b) { return bf16_bits_to_f32(b); }
template <> __device__ __forceinline__ float param_to_f32<F16>(uint32_t b) { return f16_bits_to_f32(b); }

template <typename T> __device__ __forceinline__ uint32_t f32_to_bits(float f);
template <> __device__ __forceinline__ uint32_t f32_to_bits<BF16>(float f) { return f32_to_bf16_bits(f); }
template <> __device__ __forceinline__ uint32_t f32_to_bits<F16>(float f) { return f32_to_f16_bits(f); }

// Store one fp32 result rounded once to the output dtype.
__device__ __forceinline__ void store_out(void* y, int64_t i, float v, int dt) {
  typedef __attribute__((address_space(1))) float gf32;
  typedef __attribute__((address_space(1))) uint16_t gu16;
  if (dt == DT_F32) {
    ((gf32*)y)[i] = v;
  } else if (dt == DT_BF16) {
    ((gu16*)y)[i] = (uint16_t)f32_to_bf16_bits(v);
  } else {
    ((gu16*)y)[i] = (uint16_t)f32_to_f16_bits(v);
  }
}

// 2-wide dot products with fp32 accumulation (v_dot2c_f32_bf16 / v_dot2c_f32_f16).
__device__ __forceinline__ float dot2(BF16, uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}
__device__ __forceinline__ float dot2(F16, uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
}

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ u32x4_t load16(const void* p) { return *(const u32x4_t*)p; }

// Affine rows at 2, 3, 5 or 6 bits (GPTQModel wiki "MLX Apple Silicon", Packed layouts and exact
// transcoding): each row is one little-endian bitstream, code i at stream bits [BITS i, BITS i +
// BITS), stream bit j in bit j % 32 of word j / 32.  k is a multiple of 32, so a row is made of
// 32-code chunks of exactly BITS words each.
// Code i (0..31, a constant after unrolling) of a chunk held in w[0 .. BITS-1].
template <int BITS> __device__ __forceinline__ uint32_t stream_code(const uint32_t* w, int i) {
  const int pos = BITS * i, wi = pos >> 5, sh = pos & 31;
  uint32_t v = w[wi] >> sh;
  if (sh + BITS > 32) v |= w[wi + 1] << (32 - sh);  // the code continues in the next word
  return v & ((1u << BITS) - 1u);
}

}  // namespace ql
