// kv_append: copy the new tokens' K and V rows into a contiguous or paged cache.
//
// Only the new token's projections are written; the history is never touched
// ("推理速度慢怎么办？KV Cache与Flash Attention如何加速大模型推理", section 一; the append
// of the preallocated cache in "KV Cache:推理慢的真正原因", 缓存的是什么).  The paged
// form follows the block table of "KV Cache:推理慢的真正原因" (工程优化手段 /
// PagedAttention): logical token p of a sequence sits in physical block
// table[p / 16], row p % 16.
//
// One thread moves one 16-byte chunk of a K row and the matching chunk of the
// V row.  Consecutive threads walk a row, so each wave reads and writes whole
// rows (256 B per row at d = 128 in 16-bit types).
#pragma once
#include "common.h"

namespace attn {

struct AppendArgs {
  uint4* k_cache;
  uint4* v_cache;
  const uint4* k_new;
  const uint4* v_new;
  const int32_t* cache_lens;
  const int32_t* block_table;  // nullptr -> contiguous
  int B, H_kv, n_new;
  int chunks_per_row;          // row bytes / 16
  int max_len;                 // contiguous capacity
  int max_blocks_per_seq;      // paged
  int num_blocks;              // paged
};

template <bool PAGED>
__global__ void __launch_bounds__(256) kv_append_kernel(AppendArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.B * a.H_kv * a.n_new * a.chunks_per_row;
  if (idx >= total) return;
  const int c = (int)(idx % a.chunks_per_row);
  const int64_t row = idx / a.chunks_per_row;  // row of k_new / v_new: ((b*H_kv)+h)*n_new+t
  const int t = (int)(row % a.n_new);
  const int h = (int)((row / a.n_new) % a.H_kv);
  const int b = (int)(row / ((int64_t)a.n_new * a.H_kv));

  const int start = a.cache_lens[b];
  if (start < 0) {
    if (c == 0) raise_device_error(4);
    return;
  }
  const int64_t p = (int64_t)start + t;
  int64_t dst_row;
  if (!PAGED) {
    if (p >= a.max_len) {
      if (c == 0) raise_device_error(1);
      return;
    }
    dst_row = ((int64_t)b * a.H_kv + h) * a.max_len + p;
  } else {
    const int64_t lb = p >> 4;
    if (lb >= a.max_blocks_per_seq) {
      if (c == 0) raise_device_error(1);
      return;
    }
    const int blk = a.block_table[(int64_t)b * a.max_blocks_per_seq + lb];
    if (blk < 0 || blk >= a.num_blocks) {
      if (c == 0) raise_device_error(2);
      return;
    }
    dst_row = ((int64_t)blk * a.H_kv + h) * 16 + (p & 15);
  }
  const int64_t src = row * a.chunks_per_row + c;
  const int64_t dst = dst_row * a.chunks_per_row + c;
  const uint4 kv = a.k_new[src];
  const uint4 vv = a.v_new[src];
  a.k_cache[dst] = kv;
  a.v_cache[dst] = vv;
}

// ---------------------------------------------------------------------------
// FP8 cache: append with quantization.
//
// The pages name an 8-bit KV cache as a way to halve its bytes ("KV Cache:推理慢的
// 真正原因", 工程优化手段 / quantization; the fp8 KV-cache option in
// "KV缓存与Flash注意力", 实际应用).  Stored value = E4M3(x * inv_scale): x is
// the input converted exactly to fp32, inv_scale = 1 / scale in fp32, and the
// product is rounded to the nearest OCP FP8 E4M3 value (ties to even),
// saturating at +-448; NaN stays NaN.  Dequantized value = E4M3 value * scale.

// fp32 -> OCP FP8 E4M3 code (round to nearest even, saturating)
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t s = (u >> 24) & 0x80u;
  const float a = fabsf(x);
  if (a != a) return s | 0x7Fu;        // NaN
  if (a >= 448.f) return s | 0x7Eu;    // saturate (448 = 1.75 * 2^8 is the largest finite value)
  if (a < 0.015625f) {                 // below 2^-6: subnormal grid of 2^-9
    return s | (uint32_t)__builtin_rintf(a * 512.f);  // 0 .. 8; 8 is the smallest normal
  }
  // normal: keep 3 mantissa bits, rounding the 20 dropped bits to nearest even
  const uint32_t ua = __float_as_uint(a);
  const uint32_t r = (ua + 0x7FFFFu + ((ua >> 20) & 1u)) & 0xFFF00000u;
  const int e = (int)(r >> 23) - 127;  // -6 .. 8 (a < 448 cannot round past 448)
  return s | (uint32_t)((e + 7) << 3) | ((r >> 20) & 7u);
}

template <typename TIN>
__device__ __forceinline__ float in_to_f32(const void* p, int64_t i);
template <>
__device__ __forceinline__ float in_to_f32<F32>(const void* p, int64_t i) { return static_cast<const float*>(p)[i]; }
template <>
__device__ __forceinline__ float in_to_f32<BF16>(const void* p, int64_t i) {
  return __uint_as_float((uint32_t)static_cast<const uint16_t*>(p)[i] << 16);
}
template <>
__device__ __forceinline__ float in_to_f32<F16>(const void* p, int64_t i) {
  return (float)static_cast<const _Float16*>(p)[i];
}

// int8 cache with one scale per (KV head, channel): a few keys are very large,
// so one scale for a whole tensor would magnify their error ("KV Cache:推理慢的
// 真正原因", 工程优化手段, the quantization item).  code = rint(x / s[h][c]) in
// fp32 (the quotient correctly rounded, rint ties to even), clamped to
// [-127, 127]; NaN -> 0.
__device__ __forceinline__ uint32_t f32_to_i8(float x, float s, float lim = 127.f) {
  float r = __builtin_rintf(x / s);
  r = r != r ? 0.f : fminf(fmaxf(r, -lim), lim);
  return (uint32_t)(int32_t)r & 0xFFu;
}

struct Append8Args {
  uint8_t* k_pool;
  uint8_t* v_pool;
  const void* k_new;
  const void* v_new;
  const int32_t* cache_lens;
  const int32_t* block_table;
  int B, H_kv, n_new, d;
  int max_blocks_per_seq, num_blocks;
  float k_inv, v_inv;                  // FP8: 1 / scale, in fp32
  const float* k_scales;               // int8: [H_kv][d]
  const float* v_scales;
};

// One thread quantizes 8 consecutive elements of a K row and of the V row,
// to FP8 E4M3 (I8 = false) or to int8 with per-channel scales (I8 = true).
template <typename TIN, bool I8>
__global__ void __launch_bounds__(256) kv_append_8bit_kernel(Append8Args a) {
  const int per_row = a.d / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.B * a.H_kv * a.n_new * per_row;
  if (idx >= total) return;
  const int c = (int)(idx % per_row);
  const int64_t row = idx / per_row;  // ((b*H_kv)+h)*n_new+t
  const int t = (int)(row % a.n_new);
  const int h = (int)((row / a.n_new) % a.H_kv);
  const int b = (int)(row / ((int64_t)a.n_new * a.H_kv));
  const int start = a.cache_lens[b];
  if (start < 0) {
    if (c == 0) raise_device_error(4);
    return;
  }
  const int64_t p = (int64_t)start + t;
  const int64_t lb = p >> 4;
  if (lb >= a.max_blocks_per_seq) {
    if (c == 0) raise_device_error(1);
    return;
  }
  const int blk = a.block_table[(int64_t)b * a.max_blocks_per_seq + lb];
  if (blk < 0 || blk >= a.num_blocks) {
    if (c == 0) raise_device_error(2);
    return;
  }
  const int64_t dst = (((int64_t)blk * a.H_kv + h) * 16 + (p & 15)) * a.d + 8 * c;
  const int64_t src = row * a.d + 8 * c;
  uint32_t kw[2] = {0u, 0u}, vw[2] = {0u, 0u};
  if constexpr (I8) {
    const float* ksc = a.k_scales + (int64_t)h * a.d + 8 * c;
    const float* vsc = a.v_scales + (int64_t)h * a.d + 8 * c;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kw[e >> 2] |= f32_to_i8(in_to_f32<TIN>(a.k_new, src + e), ksc[e]) << (8 * (e & 3));
      vw[e >> 2] |= f32_to_i8(in_to_f32<TIN>(a.v_new, src + e), vsc[e]) << (8 * (e & 3));
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kw[e >> 2] |= f32_to_e4m3(in_to_f32<TIN>(a.k_new, src + e) * a.k_inv) << (8 * (e & 3));
      vw[e >> 2] |= f32_to_e4m3(in_to_f32<TIN>(a.v_new, src + e) * a.v_inv) << (8 * (e & 3));
    }
  }
  *reinterpret_cast<uint2*>(a.k_pool + dst) = make_uint2(kw[0], kw[1]);
  *reinterpret_cast<uint2*>(a.v_pool + dst) = make_uint2(vw[0], vw[1]);
}

// int4 cache: the int8 rule with codes clamped to [-7, 7], two per byte
// (4-bit two's complement).  K rows: element 2i in the low nibble, 2i + 1 in
// the high one.  V: each (block, KV head) of 16 tokens x d channels is 8 d
// bytes in the order the decode's P V product reads them: 64 runs of d / 8
// bytes, run 16 g + i holding tokens 4 g .. 4 g + 3 of channels i + 16 m;
// byte 4 w + j of a run holds token 4 g + kI4VTok[j] of channel 32 w + i (low
// nibble) and 32 w + 16 + i (high nibble).  So a byte holds one token, and an
// append writes whole bytes.  One thread quantizes 32 consecutive channels of
// a token: 16 bytes of its K row, and 16 single bytes of V (channels
// 32 c + i and 32 c + 16 + i, i = 0 .. 15).
__device__ __forceinline__ constexpr int kI4VTok(int j) { return j == 1 ? 2 : j == 2 ? 1 : j; }  // self-inverse
template <typename TIN>
__global__ void __launch_bounds__(256) kv_append_int4_kernel(Append8Args a) {
  const int per_row = a.d / 32;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.B * a.H_kv * a.n_new * per_row;
  if (idx >= total) return;
  const int c = (int)(idx % per_row);
  const int64_t row = idx / per_row;  // ((b*H_kv)+h)*n_new+t
  const int t = (int)(row % a.n_new);
  const int h = (int)((row / a.n_new) % a.H_kv);
  const int b = (int)(row / ((int64_t)a.n_new * a.H_kv));
  const int start = a.cache_lens[b];
  if (start < 0) {
    if (c == 0) raise_device_error(4);
    return;
  }
  const int64_t p = (int64_t)start + t;
  const int64_t lb = p >> 4;
  if (lb >= a.max_blocks_per_seq) {
    if (c == 0) raise_device_error(1);
    return;
  }
  const int blk = a.block_table[(int64_t)b * a.max_blocks_per_seq + lb];
  if (blk < 0 || blk >= a.num_blocks) {
    if (c == 0) raise_device_error(2);
    return;
  }
  const int r = (int)(p & 15);                                   // token of the block
  const int64_t base = ((int64_t)blk * a.H_kv + h) * 8 * a.d;   // the (block, KV head)'s bytes
  const int64_t src = row * a.d + 32 * c;
  const float* ksc = a.k_scales + (int64_t)h * a.d + 32 * c;
  const float* vsc = a.v_scales + (int64_t)h * a.d + 32 * c;
  uint32_t kw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < 32; ++e)
    kw[e >> 3] |= (f32_to_i8(in_to_f32<TIN>(a.k_new, src + e), ksc[e], 7.f) & 0xFu) << (4 * (e & 7));
  *reinterpret_cast<uint4*>(a.k_pool + base + (int64_t)r * (a.d / 2) + 16 * c) = make_uint4(kw[0], kw[1], kw[2], kw[3]);
  const int64_t vrun0 = base + (int64_t)(16 * (r >> 2)) * (a.d / 8) + 4 * c + kI4VTok(r & 3);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t lo = f32_to_i8(in_to_f32<TIN>(a.v_new, src + i), vsc[i], 7.f) & 0xFu;
    const uint32_t hi = f32_to_i8(in_to_f32<TIN>(a.v_new, src + 16 + i), vsc[16 + i], 7.f) & 0xFu;
    a.v_pool[vrun0 + (int64_t)i * (a.d / 8)] = (uint8_t)(lo | (hi << 4));
  }
}

// kv_copy_blocks: duplicate whole physical blocks (every KV head) of the K and V
// pools, the copy half of copy on write when a sequence forked from a shared
// prompt first writes into the prompt's partly filled last block
// ("KV缓存与Flash注意力", 练习, prompts whose cache is shared by the completions
// that branch from it).  blockIdx.y picks the (src, dst) pair; the x dimension
// walks the block in 16-byte chunks, so each wave moves 1 KiB contiguous.
struct CopyBlocksArgs {
  uint4* k_pool;
  uint4* v_pool;
  const int32_t* pairs;      // [n_pairs][2] = (src, dst)
  int64_t chunks_per_block;  // H_kv * 16 * row bytes / 16
  int num_blocks;
};

__global__ void __launch_bounds__(256) kv_copy_blocks_kernel(CopyBlocksArgs a) {
  const int src = a.pairs[2 * blockIdx.y];
  const int dst = a.pairs[2 * blockIdx.y + 1];
  if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks) {
    if (blockIdx.x == 0 && threadIdx.x == 0) raise_device_error(2);
    return;
  }
  const int64_t s0 = (int64_t)src * a.chunks_per_block, d0 = (int64_t)dst * a.chunks_per_block;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < a.chunks_per_block;
       c += (int64_t)gridDim.x * blockDim.x) {
    const uint4 k = a.k_pool[s0 + c];
    const uint4 v = a.v_pool[s0 + c];
    a.k_pool[d0 + c] = k;
    a.v_pool[d0 + c] = v;
  }
}

}  // namespace attn
