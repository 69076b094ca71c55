"""CPU fp64 oracle for exact softmax attention with a KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (the HIP library and its Python binding) never does,
and this package imports nothing from it.

What it computes (the plain definition the tiled GPU method must reach):

    O[b, h, i, :] = sum_j softmax_j(scale * q_i . k_j) * v_j     over visible keys j
    lse[b, h, i]  = ln sum_j exp(scale * q_i . k_j)

with query head ``h`` reading KV head ``h // (H_q / H_kv)``.  Every value is the
exact fp64 upcast of the stored (rounded) input bits.

Sources, cited by page title and section:

* "推理速度慢怎么办？KV Cache与Flash Attention如何加速大模型推理" (ipipp.com):
  section 一 (append-then-attend decode step, KV-cache size formula);
  section 二 (tiles of Q / K / V, running max and normaliser, exact result).
* "KV缓存与Flash注意力" (FANDEX): KV缓存数学 (bytes per token), Flash Attention —
  分块技巧 (tile loop, running (max, sum)), 步骤1 (list-of-lists cache),
  步骤2 (online softmax over tiles), 步骤3 (naive vs cached operation counts),
  练习 (16-token blocks with a free list).
* "KV Cache:推理慢的真正原因" (cybercheems.top): 为什么需要 KV Cache (sum of i),
  缓存的是什么 (shapes, preallocated append cache), 显存账 (bytes per token),
  工程优化手段 (PagedAttention block table, GQA head sharing).

Parity status of each function is listed in the docstring of its module.
"""
from .numerics import decode_bits, kv_bytes, kv_head_of
from .attention import (one_shot, softmax_weights, tiled, splitk_merge, attention_rows)
from .brute import brute_attention
from .caches import ListCache, ContigCache, PagedCache
from .decode import cached_decode, naive_decode, decode_step, chunk_step
from .fp8 import E4M3_VALUES, e4m3_round, e4m3_value, quantize, decode_step_fp8, prefill_fp8
from .block_pool import FreeListPool, NoBlocks, blocks_for, simulate
from .int8 import (quantize_int8, dequantize_int8, decode_step_int8, quantize_int4, pack_int4, unpack_int4,
                   decode_step_int4, int4_v_position, int4_v_to_pool, int4_v_from_pool)

__all__ = [
    "decode_bits", "kv_bytes", "kv_head_of",
    "one_shot", "softmax_weights", "tiled", "splitk_merge", "attention_rows",
    "brute_attention",
    "ListCache", "ContigCache", "PagedCache",
    "cached_decode", "naive_decode", "decode_step", "chunk_step",
    "E4M3_VALUES", "e4m3_round", "e4m3_value", "quantize", "decode_step_fp8", "prefill_fp8",
    "FreeListPool", "NoBlocks", "blocks_for", "simulate",
    "quantize_int8", "dequantize_int8", "decode_step_int8", "quantize_int4", "pack_int4", "unpack_int4",
    "decode_step_int4", "int4_v_position", "int4_v_to_pool", "int4_v_from_pool",
]
