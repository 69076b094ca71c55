"""Symmetric int8 KV cache with one scale per (KV head, channel), and a decode
step over it.

Test infrastructure only (see the package docstring).

Quantizing the cache to int8 (or int4) shrinks it further; a few keys are very
large, and quantizing them with one scale for a whole tensor magnifies the
error, so the scale is kept per channel ("KV Cache:推理慢的真正原因",
工程优化手段, the quantization item; int8 and int4 caches are also named in
"推理速度慢怎么办？KV Cache与Flash Attention如何加速大模型推理", section 三).

Reading taken here: channel c of KV head h has one fp32 scale s[h, c] > 0,
fixed ahead of time (calibrated by the caller) and shared by every token; a
group of channels sharing a scale is the special case of equal entries.

    code  = clamp(rint(float32(x) / float32(s)), -127, 127)   (x converted
            exactly to float32, the quotient rounded to float32, rint ties to
            even; NaN -> 0; +-inf -> +-127)
    value = code * s

int4 (the same page and section): the same scales and rounding with codes
clamped to [-7, 7], two per byte as 4-bit two's complement.  K rows: element
2i in the low nibble and element 2i + 1 in the high nibble.  V: each (block,
KV head) of 16 tokens x d channels is 8 d bytes in the order the decode's
P V product reads them (``int4_v_position``): 64 runs of d / 8 bytes, run
16 g + i holding tokens 4 g .. 4 g + 3 of channels i, i + 16, i + 32, ...;
byte 4 w + j of a run holds token 4 g + (0, 2, 1, 3)[j] of channel
32 w + i (low nibble) and 32 w + 16 + i (high nibble).  The pool keeps the
shape [num_blocks, H_kv, 16, d / 2]; only the order of a block's bytes
differs from K's rows.

Pins (tests/test_oracle_int8.py): hand values, brute-force nearest-integer
rounding, ties, saturation, the per-channel scale selecting the right channel
and head, nibble packing, the int4 V pool's order (positions worked out by
hand, one token per byte, round trips over random bytes), and decode steps
equal to attention over the dequantized cache.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_rows
from .caches import PagedCache
from .numerics import decode_bits

INT8_MAX = 127


def quantize_int8(x_bits: np.ndarray, dtype: str, scales: np.ndarray, limit: int = INT8_MAX) -> np.ndarray:
    """Storage bits [..., H_kv, n, d] of ``dtype`` -> int8 codes in [-limit, limit],
    with scales [H_kv, d]."""
    x = decode_bits(x_bits, dtype).astype(np.float32)   # exact: every input type fits float32
    s = np.asarray(scales, dtype=np.float32)[:, None, :]  # broadcast over tokens
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        y = x / s                                        # IEEE float32 quotient
    r = np.rint(y)                                       # ties to even
    r = np.where(np.isnan(r), 0.0, r)
    return np.clip(r, -limit, limit).astype(np.int8)


def dequantize_int8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """int8 codes [H_kv, n, d] -> fp64 values code * s[h, c]."""
    return codes.astype(np.float64) * np.asarray(scales, dtype=np.float32).astype(np.float64)[:, None, :]


def decode_step_int8(cache: PagedCache, q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
                     lens: np.ndarray, scale: float, dtype: str, k_scales: np.ndarray, v_scales: np.ndarray,
                     heads=None):
    """Quantize and append the new rows into the int8 pools, then attend.

    ``cache`` holds int8 codes and is modified in place.  ``q`` [B, H_q, d] and the
    new rows [B, H_kv, n_new, d] are storage bits of ``dtype``; k_scales and
    v_scales are [H_kv, d].  Returns (O, lse) in fp64 like ``decode_step``.
    """
    B = k_new.shape[0]
    kq = np.stack([quantize_int8(k_new[b], dtype, k_scales) for b in range(B)])
    vq = np.stack([quantize_int8(v_new[b], dtype, v_scales) for b in range(B)])
    cache.append(kq, vq, lens)
    _, H_q, d = q.shape
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
        K = dequantize_int8(Kc, k_scales)[None]
        V = dequantize_int8(Vc, v_scales)[None]
        qb = decode_bits(q[b], dtype)[None, :, None, :]
        o, ls = attention_rows(qb, K, V, scale, [(0, h, 0) for h in hs])
        for r, h in enumerate(hs):
            O[b, h], L[b, h] = o[r], ls[r]
    return O, L


INT4_MAX = 7


def quantize_int4(x_bits: np.ndarray, dtype: str, scales: np.ndarray) -> np.ndarray:
    """Storage bits [..., H_kv, n, d] -> int4 codes in [-7, 7] (held in int8)."""
    return quantize_int8(x_bits, dtype, scales, INT4_MAX)


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """int4 codes [..., d] -> bytes [..., d / 2]: element 2i low nibble, 2i + 1 high."""
    c = codes.astype(np.int16) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """bytes [..., d / 2] -> int4 codes [..., d] (int8), sign-extending each nibble."""
    p = packed.astype(np.int16)
    lo, hi = p & 0xF, (p >> 4) & 0xF
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.int16)
    out[..., 0::2], out[..., 1::2] = lo, hi
    return np.where(out >= 8, out - 16, out).astype(np.int8)


_V_BYTE_OF_TOKEN = (0, 2, 1, 3)  # byte j of a 4-byte word holds token (0, 2, 1, 3)[j] of its group


def int4_v_position(t: int, c: int, d: int):
    """(byte offset, nibble) of token t (0..15), channel c (0..d-1) within one
    (block, KV head) of the int4 V pool (8 d bytes; nibble 0 low, 1 high).  The
    layout pairs channel groups c // 16, so d is a multiple of 32."""
    if d % 32 or not (0 <= t < 16 and 0 <= c < d):
        raise ValueError("int4 V pool: d must be a multiple of 32, 0 <= t < 16, 0 <= c < d")
    g, i, m = t // 4, c % 16, c // 16
    run = 16 * g + i
    return run * (d // 8) + 4 * (m // 2) + _V_BYTE_OF_TOKEN.index(t % 4), m % 2


def int4_v_to_pool(rows: np.ndarray) -> np.ndarray:
    """V bytes [..., 16, d / 2] in row order (``pack_int4`` of each token) ->
    the same codes in the pool's order, same shape."""
    codes = unpack_int4(rows).astype(np.int16) & 0xF  # [..., 16, d]
    d = codes.shape[-1]
    out = np.zeros(rows.shape[:-2] + (8 * d,), np.int16)
    for t in range(16):
        for c in range(d):
            off, hi = int4_v_position(t, c, d)
            out[..., off] |= codes[..., t, c] << (4 * hi)
    return out.astype(np.uint8).reshape(rows.shape)


def int4_v_from_pool(blocks: np.ndarray) -> np.ndarray:
    """Inverse of ``int4_v_to_pool``: V bytes in the pool's order -> row order."""
    d = 2 * blocks.shape[-1]
    flat = blocks.reshape(blocks.shape[:-2] + (8 * d,)).astype(np.int16)
    codes = np.zeros(blocks.shape[:-2] + (16, d), np.int16)
    for t in range(16):
        for c in range(d):
            off, hi = int4_v_position(t, c, d)
            codes[..., t, c] = (flat[..., off] >> (4 * hi)) & 0xF
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def decode_step_int4(cache: PagedCache, q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
                     lens: np.ndarray, scale: float, dtype: str, k_scales: np.ndarray, v_scales: np.ndarray,
                     heads=None):
    """``decode_step_int8`` over int4 pools: ``cache`` holds packed bytes
    [num_blocks, H_kv, 16, d / 2] (V in the pool's order) and is modified in place."""
    B = k_new.shape[0]
    kq = np.stack([pack_int4(quantize_int4(k_new[b], dtype, k_scales)) for b in range(B)])
    vq = np.stack([pack_int4(quantize_int4(v_new[b], dtype, v_scales)) for b in range(B)])
    rows = PagedCache(cache.k, int4_v_from_pool(cache.v), cache.table)
    rows.append(kq, vq, lens)
    cache.k[...] = rows.k
    cache.v[...] = int4_v_to_pool(rows.v)
    _, H_q, d = q.shape
    n_new = k_new.shape[2]
    O = np.full((B, H_q, d), np.nan)
    L = np.full((B, H_q), np.nan)
    wanted = heads if heads is not None else [(b, h) for b in range(B) for h in range(H_q)]
    by_b = {}
    for b, h in wanted:
        by_b.setdefault(b, []).append(h)
    for b, hs in sorted(by_b.items()):
        n = int(lens[b]) + n_new
        Kc, Vc = rows.gather(b, n)  # V back in row order
        K = dequantize_int8(unpack_int4(Kc), k_scales)[None]
        V = dequantize_int8(unpack_int4(Vc), v_scales)[None]
        qb = decode_bits(q[b], dtype)[None, :, None, :]
        o, ls = attention_rows(qb, K, V, scale, [(0, h, 0) for h in hs])
        for r, h in enumerate(hs):
            O[b, h], L[b, h] = o[r], ls[r]
    return O, L
