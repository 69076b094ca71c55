// Helpers shared by the MFMA kernels of libattn (gfx950): 16-bit packing,
// pair sums, lane exchanges, direct global -> LDS copies and FP8 widening.
#pragma once
#include <type_traits>
#include "common.h"

namespace attn {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Two fp32 values -> two 16-bit values (round to nearest even) in one register.
template <typename T>
__device__ __forceinline__ uint32_t cvt_pk(float a, float b);
template <>
__device__ __forceinline__ uint32_t cvt_pk<BF16>(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}
template <>
__device__ __forceinline__ uint32_t cvt_pk<F16>(float a, float b) {
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), f16x2_t));
}

// Sum of the two 16-bit values packed in `x`, added to `acc` (v_dot2 with 1.0).
// The normaliser of O is accumulated from the ROUNDED weights that the P V
// product uses, so numerator and denominator see the same weights (a row whose
// softmax is one-hot returns that V row exactly).  The lse, when requested,
// is taken from a separate fp32 sum of the unrounded weights.
template <typename T>
__device__ __forceinline__ float add_pair(uint32_t x, float acc);
template <>
__device__ __forceinline__ float add_pair<BF16>(uint32_t x, float acc) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x),
                                         __builtin_bit_cast(bf16x2_t, 0x3f803f80u), acc, false);
}
template <>
__device__ __forceinline__ float add_pair<F16>(uint32_t x, float acc) {
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, x), __builtin_bit_cast(f16x2_t, 0x3c003c00u), acc,
                                false);
}

constexpr float kRescaleSlack = 8.0f;  // log2 units: weights never exceed 2^8

// s_waitcnt operands (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8; a field at its maximum does not wait).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitVmcnt0 = waitcnt_vm(0);
constexpr int kWaitLgkmcnt0 = 15 | (3 << 14) | (7 << 4);

// One wave-wide global -> LDS copy: lane l moves 16 bytes from `src` to LDS
// byte address lds_base + 16 l (global_load_lds_dwordx4; lds_base is
// wave-uniform and goes through M0, which is saved and restored).  Written as
// inline assembly so that the compiler does not treat the copy as a possible
// writer of every later LDS read: completion is awaited explicitly (vmcnt)
// before the barrier that publishes the tile.
__device__ __forceinline__ void lds_copy16(const void* src, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds_base)
      : "memory");
}

// Same copy with a wave-uniform 64-bit base (SGPRs) and per-lane 32-bit byte
// offsets (global_load_lds_dwordx4 v_off, s_base): no per-lane address math.
__device__ __forceinline__ void lds_copy16(const void* sbase, uint32_t voff, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds_base)
      : "memory");
}

// max / sum of x over lanes l and l ^ 32 (v_permlane32_swap, no LDS traffic)
__device__ __forceinline__ float max_pair32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_pair32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Two FP8 E4M3 values (byte pair `HI` of word x) -> two 16-bit T values.  Every
// E4M3 value is exact in bf16 and f16, so this is a pure format change.
template <typename T, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to(uint32_t x) {
  if constexpr (std::is_same<T, BF16>::value)
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, HI));
  else
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, HI));
}
// 8 bytes of FP8 -> 8 values of T (one 16-byte vector)
template <typename T>
__device__ __forceinline__ u32x4 fp8x8_to(const u32x2 w) {
  return u32x4{fp8x2_to<T, false>(w[0]), fp8x2_to<T, true>(w[0]), fp8x2_to<T, false>(w[1]), fp8x2_to<T, true>(w[1])};
}

}  // namespace attn
