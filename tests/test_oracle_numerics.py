"""Pins of storage-bit rounding/decoding and of the KV-cache byte count."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_kv_bytes_matches_printed_figures():
    data = json.load(open(os.path.join(GOLDEN, "kv_bytes.json")))
    for c in data["cases"]:
        got = oracle.kv_bytes(c["layers"], c["kv_heads"], c["head_dim"], c["elem_bytes"],
                              batch=c["batch"], tokens=c["tokens"])
        assert got == c["bytes"], c["cite"]


def test_kv_bytes_gqa_ratio():
    """Cache size scales with H_kv / H_q: 8 KV groups for 64 query heads is 1/8."""
    mha = oracle.kv_bytes(80, 64, 128, 2, tokens=4096)
    gqa = oracle.kv_bytes(80, 8, 128, 2, tokens=4096)
    assert mha == 8 * gqa


def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F80, 0xFF80, 0x0001, 0x4600, 0x3F81],
                    dtype=np.uint16)
    got = oracle.decode_bits(bits, "bf16")
    expect = [1.0, -2.0, 0.0, -0.0, math.inf, -math.inf, 2.0 ** -133, 8192.0, 1.0 + 2.0 ** -7]
    assert got.tolist() == expect
    assert math.copysign(1.0, got[3]) == -1.0


def test_f16_decode_roundtrip():
    x = np.array([0.0, 1.0, -2.5, 65504.0, 6e-8, 8192.0], dtype=np.float16)
    assert oracle.decode_bits(x.view(np.uint16), "f16").tolist() == x.astype(np.float64).tolist()


def _nearest_bf16(x: float) -> float:
    """Brute force: the bf16 value nearest x, ties to the even mantissa."""
    f = np.float32(x)
    u = int(np.array([f]).view(np.uint32)[0])
    lo = (u >> 16) << 16
    hi = lo + (1 << 16)
    vlo = float(np.array([lo], dtype=np.uint32).view(np.float32)[0])
    vhi = float(np.array([hi & 0xFFFFFFFF], dtype=np.uint32).view(np.float32)[0])
    dlo, dhi = abs(float(f) - vlo), abs(vhi - float(f))
    if dlo < dhi:
        return vlo
    if dhi < dlo:
        return vhi
    return vlo if ((lo >> 16) & 1) == 0 else vhi


def test_bf16_rounding_ties_to_even():
    ties = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 2.0 + 2.0 ** -7,
            1.0 + 2.0 ** -8 + 2.0 ** -20, 1.0 + 2.0 ** -8 - 2.0 ** -20]
    bits = synth.f32_to_bf16_bits(np.array(ties, dtype=np.float32))
    got = oracle.decode_bits(bits, "bf16")
    assert got.tolist() == [_nearest_bf16(t) for t in ties]
    assert got[0] == 1.0 and got[1] == 1.0 + 2.0 ** -6


def test_bf16_rounding_random_against_brute():
    x = np.random.Generator(np.random.SFC64(7)).standard_normal(2000).astype(np.float32)
    got = oracle.decode_bits(synth.f32_to_bf16_bits(x), "bf16")
    assert got.tolist() == [_nearest_bf16(float(t)) for t in x]


def test_f16_rounding_is_nearest():
    x = np.random.Generator(np.random.SFC64(8)).standard_normal(500).astype(np.float32)
    got = oracle.decode_bits(synth.f32_to_f16_bits(x), "f16")
    err = np.abs(got - x.astype(np.float64))
    ulp = np.abs(np.spacing(got.astype(np.float16)).astype(np.float64))
    assert np.all(err <= ulp / 2 + 1e-300)


def test_kv_head_map():
    assert [oracle.kv_head_of(h, 64, 8) for h in (0, 7, 8, 63)] == [0, 0, 1, 7]
    with pytest.raises(ValueError):
        oracle.kv_head_of(0, 6, 4)
