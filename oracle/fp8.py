"""OCP FP8 E4M3: the value of every code, rounding to the nearest code, and a
decode step over an 8-bit paged KV cache.

Test infrastructure only (see the package docstring).

An 8-bit KV cache halves the bytes a decode step reads ("KV Cache:推理慢的真正原因",
工程优化手段 / quantization; the fp8 KV-cache option in "KV缓存与Flash注意力",
实际应用).  The format is OCP FP8 E4M3 (the "FN" variant): 1 sign bit, 4
exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds subnormals
m * 2^-9; no infinities; 0x7F / 0xFF are NaN; the largest finite value is
0x7E = 1.75 * 2^8 = 448.  One scale per tensor:

    code  = nearest E4M3 value to  float32(x) * (float32(1) / float32(scale)),
            ties to the even code (mantissa LSB 0), |.| >= 448 -> +-448, NaN -> NaN
    value = E4M3(code) * scale

FP8 prefill (the FP8 attention of FlashAttention-3 named in "KV缓存与Flash注意力",
版本演进 table and Flash Attention section): Q, K and V are E4M3 codes with one
scale each; the result is attention over the dequantized values,

    O = softmax(scale * (q_scale Q) (k_scale K)^T) (v_scale V).

Pins (tests/test_oracle_fp8.py): the format's landmark values, brute-force
nearest-value rounding on random and tie inputs, code round trips, a decode
step equal to attention over the dequantized cache, and FP8 prefill equal to
one-shot attention over dequantized values computed apart, with the scales
entering as stated.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_rows
from .caches import PagedCache
from .numerics import decode_bits


def _values() -> np.ndarray:
    v = np.empty(256)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            v[c] = np.nan
            continue
        mag = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        v[c] = -mag if s else mag
    return v


E4M3_VALUES = _values()
E4M3_MAX = 448.0
_POS = E4M3_VALUES[:127]  # codes 0x00 .. 0x7E: the non-negative finite values, increasing


def e4m3_round(y: np.ndarray) -> np.ndarray:
    """Codes of the E4M3 values nearest to float32 ``y`` (ties to the even code)."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64)
    sign = np.where(np.signbit(y), 0x80, 0).astype(np.uint8)
    a_c = np.minimum(a, E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS, a_c, side="left"), 0, 126)   # first value >= a
    lo = np.clip(hi - 1, 0, 126)
    d_hi = _POS[hi] - a_c
    d_lo = a_c - _POS[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi).astype(np.uint8)
    code = np.where(np.isnan(y), 0x7F, code).astype(np.uint8)
    return (code | sign).astype(np.uint8)


def e4m3_value(code: np.ndarray) -> np.ndarray:
    return E4M3_VALUES[np.asarray(code, dtype=np.uint8)]


def quantize(x_bits: np.ndarray, dtype: str, scale: float) -> np.ndarray:
    """Storage bits of ``dtype`` -> E4M3 codes of x / scale (the product in float32)."""
    x = decode_bits(x_bits, dtype).astype(np.float32)  # exact: every input type fits float32
    inv = np.float32(1.0) / np.float32(scale)
    return e4m3_round(x * inv)


def decode_step_fp8(cache: PagedCache, q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
                    lens: np.ndarray, scale: float, dtype: str, k_scale: float, v_scale: float,
                    heads=None):
    """Quantize and append the new rows into the 8-bit pools, then attend.

    ``cache`` holds E4M3 codes (uint8) and is modified in place.  ``q`` [B, H_q, d]
    and the new rows [B, H_kv, n_new, d] are storage bits of ``dtype``.  Returns
    (O, lse) in fp64 like ``decode_step``; keys and values are the dequantized
    codes times their scale.
    """
    cache.append(quantize(k_new, dtype, k_scale), quantize(v_new, dtype, v_scale), lens)
    B, H_q, d = q.shape
    n_new = k_new.shape[2]
    O = np.full((B, H_q, d), np.nan)
    L = np.full((B, H_q), np.nan)
    wanted = heads if heads is not None else [(b, h) for b in range(B) for h in range(H_q)]
    by_b = {}
    for b, h in wanted:
        by_b.setdefault(b, []).append(h)
    for b, hs in sorted(by_b.items()):
        n = int(lens[b]) + n_new
        Kc, Vc = cache.gather(b, n)
        K = (e4m3_value(Kc) * np.float64(k_scale))[None]
        V = (e4m3_value(Vc) * np.float64(v_scale))[None]
        qb = decode_bits(q[b], dtype)[None, :, None, :]
        o, ls = attention_rows(qb, K, V, scale, [(0, h, 0) for h in hs])
        for r, h in enumerate(hs):
            O[b, h], L[b, h] = o[r], ls[r]
    return O, L


def prefill_fp8(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_scale: float, k_scale: float, v_scale: float,
                scale: float, causal: bool, rows=None):
    """Attention over E4M3 codes q [B, H_q, N, d], k, v [B, H_kv, N, d] (uint8),
    each dequantized as code value * its scale.  Returns (O, lse) in fp64, for
    all rows or for the (b, h, i) triples in ``rows`` (as ``attention_rows``)."""
    Q = e4m3_value(q) * np.float64(q_scale)
    K = e4m3_value(k) * np.float64(k_scale)
    V = e4m3_value(v) * np.float64(v_scale)
    if rows is None:
        from .attention import one_shot
        return one_shot(Q, K, V, scale, causal=causal)
    return attention_rows(Q, K, V, scale, rows, causal=causal)
