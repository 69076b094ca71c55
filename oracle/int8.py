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
clamped to [-7, 7], stored two per byte, element 2i in the low nibble and
element 2i + 1 in the high nibble, each as 4-bit two's complement.

Pins (tests/test_oracle_int8.py): hand values, brute-force nearest-integer
rounding, ties, saturation, the per-channel scale selecting the right channel
and head, nibble packing, and decode steps equal to attention over the
dequantized cache.
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


def decode_step_int4(cache: PagedCache, q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
                     lens: np.ndarray, scale: float, dtype: str, k_scales: np.ndarray, v_scales: np.ndarray,
                     heads=None):
    """``decode_step_int8`` over int4 pools: ``cache`` holds packed bytes
    [num_blocks, H_kv, 16, d / 2] and is modified in place."""
    B = k_new.shape[0]
    kq = np.stack([pack_int4(quantize_int4(k_new[b], dtype, k_scales)) for b in range(B)])
    vq = np.stack([pack_int4(quantize_int4(v_new[b], dtype, v_scales)) for b in range(B)])
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
        K = dequantize_int8(unpack_int4(Kc), k_scales)[None]
        V = dequantize_int8(unpack_int4(Vc), v_scales)[None]
        qb = decode_bits(q[b], dtype)[None, :, None, :]
        o, ls = attention_rows(qb, K, V, scale, [(0, h, 0) for h in hs])
        for r, h in enumerate(hs):
            O[b, h], L[b, h] = o[r], ls[r]
    return O, L
