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

}  // namespace attn
