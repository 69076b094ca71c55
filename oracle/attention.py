"""Softmax attention in fp64: one-shot, tile-by-tile online softmax, split-and-merge.

Test infrastructure only (see the package docstring).

Visibility: without a causal mask every key is visible.  With it, key ``j`` is
visible to query ``i`` iff ``j <= i + (Nk - Nq)``; for prefill (``Nq == Nk``)
that is ``j <= i``, and a single decode query (``Nq == 1``) sees the whole cache.
A row with no visible key returns O = 0 and lse = -inf (never reached by the
workloads: every causal row sees its own key and every decode length is >= 1).

Pins (tests/test_oracle_attention.py):
* ``one_shot``      -- brute force in pure Python on tiny shapes; rows of the
                       softmax sum to 1; constant V; zero query (uniform weights,
                       lse = ln #keys); one visible key; dominant key; key/value
                       permutation invariance; torch's CPU fp64 attention.
* ``tiled``         -- equals ``one_shot`` for every tile size (the pages' claim
                       that the tiled method is exact).
* ``splitk_merge``  -- equals ``one_shot`` for every split size.
* ``attention_rows``-- equals the matching rows of ``one_shot``.
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

from .numerics import kv_head_of


def _visible(Nq: int, Nk: int, causal: bool) -> np.ndarray:
    """Boolean [Nq, Nk] mask of visible keys."""
    if not causal:
        return np.ones((Nq, Nk), dtype=bool)
    i = np.arange(Nq)[:, None]
    j = np.arange(Nk)[None, :]
    return j <= i + (Nk - Nq)


def _softmax_attend(s: np.ndarray, vis: np.ndarray, V: np.ndarray):
    """Plain softmax over the visible entries of each row of ``s``, then ``P @ V``.

    The row maximum is subtracted before exponentiating; it cancels in the
    ratio and only keeps ``exp`` in range.
    """
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    has = np.isfinite(m)
    m_safe = np.where(has, m, 0.0)
    e = np.where(vis, np.exp(s - m_safe[:, None]), 0.0)
    l = e.sum(axis=1)
    l_safe = np.where(has, l, 1.0)
    P = e / l_safe[:, None]
    O = P @ V
    lse = np.where(has, m_safe + np.log(l_safe), -np.inf)
    O[~has] = 0.0
    return O, lse, P


def one_shot(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
             causal: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """Standard attention: S = scale*Q K^T, P = softmax(S), O = P V, per (b, h_q).

    This is the three-step computation that "KV缓存与Flash注意力" (Flash
    Attention — 分块技巧) contrasts with the tiled kernel, and the per-step
    attention of the decode code in "推理速度慢怎么办？..." section 一 (scores
    scaled by 1/sqrt(head_dim), softmax, weighted sum of V).

    q: [B, H_q, Nq, d]; k, v: [B, H_kv, Nk, d]; all fp64.
    Returns O [B, H_q, Nq, d] and lse [B, H_q, Nq] (natural log).
    """
    B, H_q, Nq, d = q.shape
    _, H_kv, Nk, _ = k.shape
    vis = _visible(Nq, Nk, causal)
    O = np.zeros((B, H_q, Nq, v.shape[-1]))
    lse = np.zeros((B, H_q, Nq))
    for b in range(B):
        for h in range(H_q):
            g = kv_head_of(h, H_q, H_kv)
            s = scale * (q[b, h] @ k[b, g].T)
            O[b, h], lse[b, h], _ = _softmax_attend(s, vis, v[b, g])
    return O, lse


def softmax_weights(q: np.ndarray, k: np.ndarray, scale: float,
                    causal: bool = False) -> np.ndarray:
    """The attention weights P [B, H_q, Nq, Nk] of ``one_shot`` (masked entries 0)."""
    B, H_q, Nq, d = q.shape
    _, H_kv, Nk, _ = k.shape
    vis = _visible(Nq, Nk, causal)
    P = np.zeros((B, H_q, Nq, Nk))
    dummy_v = np.zeros((Nk, 1))
    for b in range(B):
        for h in range(H_q):
            g = kv_head_of(h, H_q, H_kv)
            s = scale * (q[b, h] @ k[b, g].T)
            P[b, h] = _softmax_attend(s, vis, dummy_v)[2]
    return P


def tiled(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
          causal: bool = False, tile: int = 4) -> Tuple[np.ndarray, np.ndarray]:
    """Online softmax over key tiles: the method the GPU kernels implement.

    Follows the running-max / running-sum loop of "KV缓存与Flash注意力" 步骤2
    (分块softmax), generalised with a scale and a mask and run for all query rows
    of a head at once.  Per row the state is (m, l, acc); for each tile of keys:

        m' = max(m, max_j s_j)
        alpha = exp(m - m')            (0 while m is still -inf)
        p_j = exp(s_j - m')            (0 for masked keys)
        l = alpha * l + sum_j p_j
        acc = alpha * acc + sum_j p_j v_j
        m = m'

    and at the end O = acc / l, lse = m + ln l.  Carrying (m, l) across tiles
    makes the final normalisation exact ("推理速度慢怎么办？..." section 二;
    "KV缓存与Flash注意力", 数值技巧), so this equals ``one_shot`` up to rounding.
    """
    if tile < 1:
        raise ValueError("tile must be >= 1")
    B, H_q, Nq, d = q.shape
    _, H_kv, Nk, dv = v.shape
    vis = _visible(Nq, Nk, causal)
    O = np.zeros((B, H_q, Nq, dv))
    lse = np.zeros((B, H_q, Nq))
    for b in range(B):
        for h in range(H_q):
            g = kv_head_of(h, H_q, H_kv)
            m = np.full(Nq, -np.inf)
            l = np.zeros(Nq)
            acc = np.zeros((Nq, dv))
            for start in range(0, Nk, tile):
                stop = min(Nk, start + tile)
                s = scale * (q[b, h] @ k[b, g, start:stop].T)
                s = np.where(vis[:, start:stop], s, -np.inf)
                m_new = np.maximum(m, s.max(axis=1))
                alpha = np.where(np.isfinite(m), np.exp(m - np.where(np.isfinite(m_new), m_new, 0.0)), 0.0)
                base = np.where(np.isfinite(m_new), m_new, 0.0)
                p = np.where(np.isfinite(s), np.exp(s - base[:, None]), 0.0)
                l = alpha * l + p.sum(axis=1)
                acc = alpha[:, None] * acc + p @ v[b, g, start:stop]
                m = m_new
            has = l > 0
            O[b, h] = np.where(has[:, None], acc / np.where(has, l, 1.0)[:, None], 0.0)
            lse[b, h] = np.where(has, m + np.log(np.where(has, l, 1.0)), -np.inf)
    return O, lse


def splitk_merge(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                 split: int, causal: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """Attention over key chunks of ``split`` keys, merged through their lse.

    Each chunk c gives a normalised partial (O_c, lse_c) from ``one_shot``.  With
    M = max_c lse_c and w_c = exp(lse_c - M):  O = sum_c w_c O_c / sum_c w_c and
    lse = M + ln sum_c w_c.  This is the same (max, sum) carry as the tile loop,
    at chunk granularity; chunks with no visible key (lse_c = -inf) weigh 0.
    """
    if split < 1:
        raise ValueError("split must be >= 1")
    B, H_q, Nq, d = q.shape
    Nk = k.shape[2]
    vis = _visible(Nq, Nk, causal)
    parts = []
    for start in range(0, Nk, split):
        stop = min(Nk, start + split)
        # one_shot on the chunk, with the chunk's slice of the global mask
        kc, vc = k[:, :, start:stop], v[:, :, start:stop]
        Oc = np.zeros((B, H_q, Nq, v.shape[-1]))
        lc = np.zeros((B, H_q, Nq))
        for b in range(B):
            for h in range(H_q):
                g = kv_head_of(h, H_q, k.shape[1])
                s = scale * (q[b, h] @ kc[b, g].T)
                Oc[b, h], lc[b, h], _ = _softmax_attend(s, vis[:, start:stop], vc[b, g])
        parts.append((Oc, lc))
    L = np.stack([p[1] for p in parts])            # [S, B, H, Nq]
    M = L.max(axis=0)
    has = np.isfinite(M)
    Msafe = np.where(has, M, 0.0)
    w = np.where(np.isfinite(L), np.exp(L - Msafe[None]), 0.0)
    wsum = w.sum(axis=0)
    num = sum(w[i][..., None] * parts[i][0] for i in range(len(parts)))
    O = np.where(has[..., None], num / np.where(has, wsum, 1.0)[..., None], 0.0)
    lse = np.where(has, Msafe + np.log(np.where(has, wsum, 1.0)), -np.inf)
    return O, lse


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                   rows: Iterable[Tuple[int, int, int]], causal: bool = False,
                   kv_lens: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """``one_shot`` for selected rows (b, h_q, i) only, for sampling large inputs.

    ``q`` [B, H_q, Nq, d] and ``k``, ``v`` [B, H_kv, Nk, d] may be any array type
    that slices to fp64-convertible arrays (e.g. stored bits decoded lazily by
    the caller).  ``kv_lens[b]``, when given, limits sequence b to its first
    ``kv_lens[b]`` keys.
    """
    rows = list(rows)
    B, H_q, Nq, d = q.shape
    H_kv, Nk = k.shape[1], k.shape[2]
    out = np.zeros((len(rows), v.shape[-1]))
    lse = np.zeros(len(rows))
    for r, (b, h, i) in enumerate(rows):
        g = kv_head_of(h, H_q, H_kv)
        nk = Nk if kv_lens is None else int(kv_lens[b])
        vis = _visible(Nq, nk, causal)[i:i + 1]
        K = np.asarray(k[b, g, :nk], dtype=np.float64)
        V = np.asarray(v[b, g, :nk], dtype=np.float64)
        s = scale * (np.asarray(q[b, h, i:i + 1], dtype=np.float64) @ K.T)
        o, ls, _ = _softmax_attend(s, vis, V)
        out[r], lse[r] = o[0], ls[0]
    return out, lse
