"""Brute-force attention in pure Python (``math.exp``, ``math.fsum``) for tiny inputs.

Test infrastructure only (see the package docstring).  Written element by
element from the definition so that it shares nothing with the numpy routines
it checks: for each query row the scores are scaled dot products, the weights
are exp(score) / sum exp(score) over visible keys, and the output is the
weighted sum of value rows.  Exact sums use ``math.fsum``.
"""
from __future__ import annotations

import math
from typing import List, Tuple


def brute_attention(q, k, v, scale: float, causal: bool = False) -> Tuple[list, list]:
    """q: nested lists [B][H_q][Nq][d]; k, v: [B][H_kv][Nk][d].

    Returns (O, lse) as nested lists [B][H_q][Nq][d] and [B][H_q][Nq].
    Query head h reads KV head h * H_kv // H_q (contiguous groups).
    """
    B, H_q, Nq = len(q), len(q[0]), len(q[0][0])
    H_kv, Nk = len(k[0]), len(k[0][0])
    G = H_q // H_kv
    O: List = []
    LSE: List = []
    for b in range(B):
        Ob, Lb = [], []
        for h in range(H_q):
            g = h // G
            Oh, Lh = [], []
            for i in range(Nq):
                keys = [j for j in range(Nk) if (not causal) or j <= i + (Nk - Nq)]
                if not keys:
                    Oh.append([0.0] * len(v[0][0][0]))
                    Lh.append(-math.inf)
                    continue
                s = {j: scale * math.fsum(a * c for a, c in zip(q[b][h][i], k[b][g][j]))
                     for j in keys}
                top = max(s.values())
                ex = {j: math.exp(s[j] - top) for j in keys}
                den = math.fsum(ex.values())
                row = [math.fsum(ex[j] * v[b][g][j][c] for j in keys) / den
                       for c in range(len(v[0][0][0]))]
                Oh.append(row)
                Lh.append(top + math.log(den))
            Ob.append(Oh)
            Lb.append(Lh)
        O.append(Ob)
        LSE.append(Lb)
    return O, LSE
