"""Host block pool of a paged KV cache (the ``attn_block_pool_*`` calls of libattn).

Rows are numpy int32 arrays of ``max_blocks`` entries (one sequence's row of the
block table, -1 = unassigned); a table is a C-contiguous int32 array
[B, max_blocks] whose rows are such rows.  The pool changes them in place.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import numpy as np

from . import AttnError, lib

NO_BLOCKS = 5


class NoBlocks(AttnError):
    """The pool cannot meet a reservation (nothing was changed)."""


def _row(a: np.ndarray, name: str) -> int:
    if not isinstance(a, np.ndarray) or a.dtype != np.int32 or not a.flags.c_contiguous:
        raise ValueError(f"{name} must be a C-contiguous numpy int32 array")
    return a.ctypes.data


class BlockPool:
    """num_blocks physical blocks of 16 tokens, handed out from a free-list stack."""

    def __init__(self, num_blocks: int):
        self._L = lib()
        self._h = self._L.attn_block_pool_create(int(num_blocks))
        if not self._h:
            raise AttnError("attn_block_pool_create", 1, self._L.attn_last_error().decode())
        self.num_blocks = int(num_blocks)

    def close(self) -> None:
        if self._h:
            self._L.attn_block_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, fn: str, rc: int) -> None:
        if rc == NO_BLOCKS:
            raise NoBlocks(fn, rc, self._L.attn_last_error().decode())
        if rc != 0:
            raise AttnError(fn, rc, self._L.attn_last_error().decode())

    def free_blocks(self) -> int:
        return int(self._L.attn_block_pool_free_blocks(self._h))

    def holders(self, block: int) -> int:
        return int(self._L.attn_block_pool_holders(self._h, int(block)))

    def reserve(self, row: np.ndarray, cur_len: int, new_len: int) -> Optional[Tuple[int, int]]:
        """Cover new_len tokens; returns the (old, new) pair to copy, or None."""
        pair = np.empty(2, dtype=np.int32)
        rc = self._L.attn_block_pool_reserve(self._h, _row(row, "row"), row.shape[-1], int(cur_len), int(new_len),
                                             pair.ctypes.data)
        self._check("attn_block_pool_reserve", rc)
        return None if pair[0] < 0 else (int(pair[0]), int(pair[1]))

    def reserve_batch(self, table: np.ndarray, cur_lens: np.ndarray, new_lens: np.ndarray):
        """Reserve for every row of ``table``; returns (n_done, pairs [n_copies, 2])
        and raises NoBlocks (with ``n_done`` set on the exception) when a row fails."""
        B, mb = table.shape
        cur = np.ascontiguousarray(cur_lens, dtype=np.int32)
        new = np.ascontiguousarray(new_lens, dtype=np.int32)
        if cur.shape != (B,) or new.shape != (B,):
            raise ValueError("cur_lens and new_lens must be [B]")
        pairs = np.empty((max(B, 1), 2), dtype=np.int32)
        n_copies, n_done = ctypes.c_int(0), ctypes.c_int(0)
        rc = self._L.attn_block_pool_reserve_batch(self._h, _row(table, "table"), B, mb, cur.ctypes.data,
                                                   new.ctypes.data, pairs.ctypes.data, ctypes.byref(n_copies),
                                                   ctypes.byref(n_done))
        try:
            self._check("attn_block_pool_reserve_batch", rc)
        except AttnError as e:
            e.n_done = n_done.value
            e.pairs = pairs[:n_copies.value].copy()
            raise
        return n_done.value, pairs[:n_copies.value].copy()

    def release(self, row: np.ndarray, length: int) -> None:
        rc = self._L.attn_block_pool_release(self._h, _row(row, "row"), row.shape[-1], int(length))
        self._check("attn_block_pool_release", rc)

    def fork(self, src: np.ndarray, dst: np.ndarray, length: int) -> None:
        if dst.shape[-1] != src.shape[-1]:
            raise ValueError("src and dst rows must have the same length")
        rc = self._L.attn_block_pool_fork(self._h, _row(src, "src"), _row(dst, "dst"), src.shape[-1], int(length))
        self._check("attn_block_pool_fork", rc)
