// Device-side helpers shared by the kernels of libattn (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Element tags.  Storage is raw bits; arithmetic is fp32.
struct F32 {
  using storage = float;
  static constexpr int kBytes = 4;
};
struct F16 {
  using storage = uint16_t;
  static constexpr int kBytes = 2;
};
struct BF16 {
  using storage = uint16_t;
  static constexpr int kBytes = 2;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  _Float16 h;
  uint16_t s = (uint16_t)b;
  __builtin_memcpy(&h, &s, 2);
  return (float)h;
}

// Round-to-nearest-even conversions from fp32 to 16-bit storage bits.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 h = (__bf16)x;
  uint16_t s;
  __builtin_memcpy(&s, &h, 2);
  return s;
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  _Float16 h = (_Float16)x;
  uint16_t s;
  __builtin_memcpy(&s, &h, 2);
  return s;
}

template <typename T>
__device__ __forceinline__ float load_elem(const void* p, size_t i);
template <>
__device__ __forceinline__ float load_elem<F32>(const void* p, size_t i) {
  return static_cast<const float*>(p)[i];
}
template <>
__device__ __forceinline__ float load_elem<F16>(const void* p, size_t i) {
  return f16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
}
template <>
__device__ __forceinline__ float load_elem<BF16>(const void* p, size_t i) {
  return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
}

template <typename T>
__device__ __forceinline__ void store_elem(void* p, size_t i, float x);
template <>
__device__ __forceinline__ void store_elem<F32>(void* p, size_t i, float x) {
  static_cast<float*>(p)[i] = x;
}
template <>
__device__ __forceinline__ void store_elem<F16>(void* p, size_t i, float x) {
  static_cast<uint16_t*>(p)[i] = f32_to_f16_bits(x);
}
template <>
__device__ __forceinline__ void store_elem<BF16>(void* p, size_t i, float x) {
  static_cast<uint16_t*>(p)[i] = f32_to_bf16_bits(x);
}

// Pack two fp32 values into two 16-bit storage elements (lo = first).
template <typename T>
__device__ __forceinline__ uint32_t pack2(float a, float b);
template <>
__device__ __forceinline__ uint32_t pack2<BF16>(float a, float b) {
  return (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
}
template <>
__device__ __forceinline__ uint32_t pack2<F16>(float a, float b) {
  return (uint32_t)f32_to_f16_bits(a) | ((uint32_t)f32_to_f16_bits(b) << 16);
}

// Device error flags (bit values of enum attn_device_error in attn.h).
__device__ unsigned int g_device_errors;

__device__ __forceinline__ void raise_device_error(unsigned int flag) {
  atomicOr(&g_device_errors, flag);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lane exchange across the wave (ds_bpermute based).
__device__ __forceinline__ float xor_shfl(float v, int mask) { return __shfl_xor(v, mask, 64); }

}  // namespace attn
