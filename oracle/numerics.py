"""Storage-bit decoding, the GQA head map and the KV-cache byte count.

Test infrastructure only (see the package docstring).

Pins:
* ``decode_bits`` -- pinned by exact round trips against numpy's float16 and by
  hand-written bfloat16 bit patterns (tests/test_oracle_numerics.py).
* ``kv_bytes`` -- pinned by the byte counts the pages print
  (tests/golden/kv_bytes.json).
* ``kv_head_of`` -- pinned by the GQA-equals-repeated-MHA reduction.
"""
from __future__ import annotations

import numpy as np


def decode_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of stored elements.

    ``f32`` arrays are float32 values; ``f16`` / ``bf16`` arrays are uint16 bit
    patterns.  bfloat16 is the upper 16 bits of an IEEE binary32, so its value
    is the binary32 whose low half is zero.
    """
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(x, dtype=np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        wide = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return wide.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def kv_head_of(h_q: int, H_q: int, H_kv: int) -> int:
    """KV head read by query head ``h_q``.

    Grouped-query attention lets several query heads share one K/V head
    ("KV Cache:推理慢的真正原因", 工程优化手段 / 2. GQA: 64 query heads over 8
    KV groups).  Groups are contiguous runs of ``H_q / H_kv`` query heads.
    """
    if H_q % H_kv != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    return h_q // (H_q // H_kv)


def kv_bytes(layers: int, kv_heads: int, head_dim: int, elem_bytes: int,
             batch: int = 1, tokens: int = 1) -> int:
    """Bytes a KV cache holds: K and V, for every layer, KV head, token and batch row.

    All three pages give this product, each with a different subset of factors
    (section 一 of "推理速度慢怎么办？..." lists batch, layers, length, heads, head
    dim and element size; "KV缓存与Flash注意力" KV缓存数学 gives the per-layer,
    per-token figure; "KV Cache:推理慢的真正原因" 显存账 the per-token figure over
    all layers).  They agree once the head count is read as the number of K/V
    heads.
    """
    return 2 * batch * layers * tokens * kv_heads * head_dim * elem_bytes
