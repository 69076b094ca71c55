"""Incremental decoding: a cached decoder, a recompute-everything decoder, one decode step.

Test infrastructure only (see the package docstring).

* ``cached_decode`` -- at every step append the new token's K/V to a
  ``ListCache`` and attend the step's query to everything cached, including the
  token just appended ("推理速度慢怎么办？..." section 一: concatenate, then
  scores, softmax, weighted sum).  One K/V row is produced per step.
* ``naive_decode`` -- with no cache, every step rebuilds the K/V rows of the
  whole prefix from the token stream, then attends ("KV缓存与Flash注意力",
  问题所在 and 步骤3; "KV Cache:推理慢的真正原因", 为什么需要 KV Cache).  Step t
  (1-based) produces t rows, n(n+1)/2 in all.  Without model weights, "rebuilding"
  a row means copying that step's K/V vector afresh, which is what we count.
* ``decode_step`` -- one batched decode step against a ``ContigCache`` or
  ``PagedCache``: append ``n_new`` tokens, then attend the single query of each
  head to ``lens[b] + n_new`` keys.
* ``chunk_step`` -- a chunk of ``n_new`` new tokens per sequence with a query
  each (prefix reuse, "KV缓存与Flash注意力" 实际应用 and 练习; a multi-token
  append as in the cache class of "KV Cache:推理慢的真正原因", 缓存的是什么):
  append the chunk, then query t of sequence b, which is token ``lens[b] + t``,
  attends to keys ``0 .. lens[b] + t`` (causal) or to all ``lens[b] + n_new``.

Pins: the two decoders agree bit for bit and produce 5050 vs 100 rows at
n = 100 (tests/golden/op_counts.json); a decode step equals the matching row of
causal prefill over the whole sequence; a chunk step equals the matching rows
of causal prefill over the whole sequence, reduces to a decode step at
n_new = 1 and to plain prefill at an empty prefix (tests/test_oracle_decode.py).
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np

from .attention import one_shot, attention_rows
from .caches import ContigCache, ListCache, PagedCache
from .numerics import decode_bits, kv_head_of


def cached_decode(qs: List[np.ndarray], ks: List[np.ndarray], vs: List[np.ndarray],
                  scale: float) -> Tuple[np.ndarray, int]:
    """qs[t]: [H_q, d]; ks[t], vs[t]: [H_kv, d] (fp64).  Returns ([T, H_q, d], rows made)."""
    H_q = qs[0].shape[0]
    H_kv = ks[0].shape[0]
    cache = ListCache(1, H_kv)
    outs = []
    produced = 0
    for q, k, v in zip(qs, ks, vs):
        for g in range(H_kv):
            cache.append(0, g, k[g], v[g])
        produced += 1
        o = np.zeros((H_q, q.shape[1]))
        for h in range(H_q):
            g = kv_head_of(h, H_q, H_kv)
            Kl, Vl = cache.read(0, g)
            K = np.stack(Kl)[None, None]
            V = np.stack(Vl)[None, None]
            o[h] = one_shot(q[h][None, None, None], K, V, scale)[0][0, 0, 0]
        outs.append(o)
    return np.stack(outs), produced


def naive_decode(qs: List[np.ndarray], ks: List[np.ndarray], vs: List[np.ndarray],
                 scale: float) -> Tuple[np.ndarray, int]:
    """Same contract as ``cached_decode``, recomputing the prefix rows every step."""
    H_q = qs[0].shape[0]
    H_kv = ks[0].shape[0]
    outs = []
    produced = 0
    for t, q in enumerate(qs):
        K = np.stack([np.array(ks[i], copy=True) for i in range(t + 1)], axis=1)
        V = np.stack([np.array(vs[i], copy=True) for i in range(t + 1)], axis=1)
        produced += t + 1
        o = np.zeros((H_q, q.shape[1]))
        for h in range(H_q):
            g = kv_head_of(h, H_q, H_kv)
            o[h] = one_shot(q[h][None, None, None], K[g][None, None], V[g][None, None],
                            scale)[0][0, 0, 0]
        outs.append(o)
    return np.stack(outs), produced


def decode_step(cache, q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
                lens: np.ndarray, scale: float, dtype: str, heads=None):
    """Append then attend, on storage bits.

    ``cache`` is a ``ContigCache`` or ``PagedCache`` (modified in place: it ends
    up holding the expected append image).  ``q`` [B, H_q, d] and the new rows
    [B, H_kv, n_new, d] are storage bits.  ``heads`` optionally restricts the
    output to a list of (b, h_q) pairs.  Returns (O, lse) in fp64: [B, H_q, d]
    and [B, H_q] (rows not requested stay NaN).
    """
    cache.append(k_new, v_new, lens)
    B, H_q, d = q.shape
    H_kv = k_new.shape[1]
    n_new = k_new.shape[2]
    O = np.full((B, H_q, d), np.nan)
    L = np.full((B, H_q), np.nan)
    wanted = heads if heads is not None else [(b, h) for b in range(B) for h in range(H_q)]
    by_b = {}
    for b, h in wanted:
        by_b.setdefault(b, []).append(h)
    for b, hs in sorted(by_b.items()):
        n = int(lens[b]) + n_new
        if isinstance(cache, PagedCache):
            Kb, Vb = cache.gather(b, n)
        else:
            Kb, Vb = cache.view(b, n)
        K = decode_bits(Kb, dtype)[None]
        V = decode_bits(Vb, dtype)[None]
        qb = decode_bits(q[b], dtype)[None, :, None, :]
        rows = [(0, h, 0) for h in hs]
        o, ls = attention_rows(qb, K, V, scale, rows)
        for r, h in enumerate(hs):
            O[b, h], L[b, h] = o[r], ls[r]
    return O, L


def chunk_step(cache, q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
               lens: np.ndarray, scale: float, dtype: str, causal: bool = True, rows=None):
    """Append a chunk of ``n_new`` tokens per sequence, then attend its queries.

    ``cache`` is a ``ContigCache`` or ``PagedCache`` (modified in place).
    ``q`` [B, H_q, n_new, d] and the new rows [B, H_kv, n_new, d] are storage
    bits; query t of sequence b is token ``lens[b] + t``.  ``rows`` optionally
    restricts the output to a list of (b, h_q, t).  Returns (O, lse) in fp64:
    [B, H_q, n_new, d] and [B, H_q, n_new] (rows not requested stay NaN).
    """
    cache.append(k_new, v_new, lens)
    B, H_q, n_new, d = q.shape
    O = np.full((B, H_q, n_new, d), np.nan)
    L = np.full((B, H_q, n_new), np.nan)
    wanted = rows if rows is not None else [(b, h, t) for b in range(B) for h in range(H_q)
                                            for t in range(n_new)]
    by_b = {}
    for b, h, t in wanted:
        by_b.setdefault(b, []).append((h, t))
    for b, hts in sorted(by_b.items()):
        n = int(lens[b]) + n_new
        if isinstance(cache, PagedCache):
            Kb, Vb = cache.gather(b, n)
        else:
            Kb, Vb = cache.view(b, n)
        K = decode_bits(Kb, dtype)[None]
        V = decode_bits(Vb, dtype)[None]
        qb = decode_bits(q[b], dtype)[None]
        # Nq = n_new queries against Nk = n keys: with the causal mask, query t
        # sees keys j <= t + (n - n_new) = lens[b] + t
        o, ls = attention_rows(qb, K, V, scale, [(0, h, t) for h, t in hts], causal=causal)
        for r, (h, t) in enumerate(hts):
            O[b, h, t], L[b, h, t] = o[r], ls[r]
    return O, L
