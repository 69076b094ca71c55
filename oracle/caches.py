"""KV-cache models: list of vectors, preallocated contiguous buffer, paged pool.

Test infrastructure only (see the package docstring).  Appends move raw storage
bits (uint16 for f16/bf16, float32 for f32) by index, so an append image is
bit-exact by construction.

* ``ListCache`` -- one growing list of K and of V vectors per (layer, head),
  as in "KV缓存与Flash注意力" 步骤1 (KV缓存).
* ``ContigCache`` -- a preallocated ``[B, H_kv, max_len, d]`` buffer written at
  ``[start, start + n_new)``, as in the cache class of "KV Cache:推理慢的真正原因"
  (缓存的是什么), with a length per sequence instead of one shared length, and an
  overflow check the page's class does not have.
* ``PagedCache`` -- a pool of 16-token physical blocks ``[num_blocks, H_kv, 16, d]``
  and a per-sequence block table mapping logical block j to a physical block
  ("KV Cache:推理慢的真正原因", 工程优化手段 / 1. PagedAttention;
  "KV缓存与Flash注意力", 练习).  Token p of sequence b lives in block
  ``table[b][p // 16]`` at row ``p % 16``; -1 marks an unassigned entry.

Pins: append images are compared byte for byte with hand-computed images and
with untouched sentinel bytes; gathering a pool through its table reproduces
the contiguous cache bit for bit; the identity table is a plain reshape
(tests/test_oracle_caches.py).
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np


class ListCache:
    """Per (layer, head) lists of K and V vectors; append one vector at a time."""

    def __init__(self, n_layers: int, n_heads: int):
        self.K: List[List[list]] = [[[] for _ in range(n_heads)] for _ in range(n_layers)]
        self.V: List[List[list]] = [[[] for _ in range(n_heads)] for _ in range(n_layers)]

    def append(self, layer: int, head: int, k, v) -> None:
        self.K[layer][head].append(np.array(k, copy=True))
        self.V[layer][head].append(np.array(v, copy=True))

    def read(self, layer: int, head: int) -> Tuple[list, list]:
        return self.K[layer][head], self.V[layer][head]


class ContigCache:
    """Preallocated ``[B, H_kv, max_len, d]`` K and V buffers (storage bits)."""

    def __init__(self, k: np.ndarray, v: np.ndarray):
        if k.shape != v.shape or k.ndim != 4:
            raise ValueError("k and v must share a [B, H_kv, max_len, d] shape")
        self.k = np.array(k, copy=True)
        self.v = np.array(v, copy=True)

    @property
    def max_len(self) -> int:
        return self.k.shape[2]

    def append(self, k_new: np.ndarray, v_new: np.ndarray, cache_lens) -> None:
        """Write ``k_new[b, h, t]`` to position ``cache_lens[b] + t``.

        ``cache_lens`` is read, not advanced: the caller owns the lengths.
        Raises if a position falls outside ``[0, max_len)``.
        """
        B, H, n_new, d = k_new.shape
        for b in range(B):
            start = int(cache_lens[b])
            if start < 0 or start + n_new > self.max_len:
                raise IndexError(f"sequence {b}: positions [{start}, {start + n_new}) "
                                 f"outside a cache of {self.max_len}")
            for h in range(H):
                for t in range(n_new):
                    self.k[b, h, start + t] = k_new[b, h, t]
                    self.v[b, h, start + t] = v_new[b, h, t]

    def view(self, b: int, length: int) -> Tuple[np.ndarray, np.ndarray]:
        """The first ``length`` tokens of sequence b: two [H_kv, length, d] arrays."""
        return self.k[b, :, :length], self.v[b, :, :length]


class PagedCache:
    """A pool of fixed-size blocks plus a block table (storage bits)."""

    def __init__(self, k_pool: np.ndarray, v_pool: np.ndarray, block_table: np.ndarray,
                 block_size: int = 16):
        if k_pool.shape != v_pool.shape or k_pool.ndim != 4:
            raise ValueError("pools must share a [num_blocks, H_kv, block, d] shape")
        if k_pool.shape[2] != block_size:
            raise ValueError("pool block dimension must equal block_size")
        self.k = np.array(k_pool, copy=True)
        self.v = np.array(v_pool, copy=True)
        self.table = np.asarray(block_table, dtype=np.int64)
        self.bs = block_size

    @property
    def num_blocks(self) -> int:
        return self.k.shape[0]

    def locate(self, b: int, p: int) -> Tuple[int, int]:
        """Physical (block, row) of logical token p of sequence b."""
        j = p // self.bs
        if p < 0 or j >= self.table.shape[1]:
            raise IndexError(f"token {p} of sequence {b} beyond the block table")
        blk = int(self.table[b, j])
        if blk < 0 or blk >= self.num_blocks:
            raise IndexError(f"sequence {b} logical block {j} maps to invalid block {blk}")
        return blk, p % self.bs

    def append(self, k_new: np.ndarray, v_new: np.ndarray, cache_lens) -> None:
        """Write ``k_new[b, h, t]`` to the slot of logical token ``cache_lens[b] + t``."""
        B, H, n_new, d = k_new.shape
        for b in range(B):
            for t in range(n_new):
                blk, row = self.locate(b, int(cache_lens[b]) + t)
                for h in range(H):
                    self.k[blk, h, row] = k_new[b, h, t]
                    self.v[blk, h, row] = v_new[b, h, t]

    def gather(self, b: int, length: int) -> Tuple[np.ndarray, np.ndarray]:
        """The first ``length`` tokens of sequence b as [H_kv, length, d] arrays."""
        H, d = self.k.shape[1], self.k.shape[3]
        K = np.empty((H, length, d), dtype=self.k.dtype)
        V = np.empty((H, length, d), dtype=self.v.dtype)
        for p in range(length):
            blk, row = self.locate(b, p)
            K[:, p] = self.k[blk, :, row]
            V[:, p] = self.v[blk, :, row]
        return K, V
