"""Pins of the FP8 E4M3 oracle: format landmarks, nearest-value rounding, decode over dequantized codes."""
import math

import numpy as np

import oracle
import synth


def test_format_landmarks():
    v = oracle.E4M3_VALUES
    assert v[0x7E] == 448.0                       # largest finite: 1.75 * 2^8
    assert v[0x08] == 2.0 ** -6                   # smallest normal
    assert v[0x01] == 2.0 ** -9                   # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9               # largest subnormal
    assert v[0x38] == 1.0 and v[0x39] == 1.125 and v[0xB8] == -1.0
    assert math.isnan(v[0x7F]) and math.isnan(v[0xFF])
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and math.copysign(1, v[0x80]) == -1
    finite = v[:0x7F]
    assert np.all(np.diff(finite) > 0)            # codes 0 .. 0x7E increase
    assert np.sum(np.isnan(v)) == 2 and not np.any(np.isinf(v))


def test_codes_round_trip():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    back = oracle.e4m3_round(oracle.e4m3_value(codes).astype(np.float32))
    assert np.array_equal(back, codes)


def test_rounding_against_brute_force():
    r = np.random.Generator(np.random.SFC64(5))
    y = np.concatenate([r.standard_normal(3000) * s for s in (0.003, 0.05, 1.0, 40.0, 300.0)]).astype(np.float32)
    got = oracle.e4m3_round(y)
    finite = [(c, oracle.E4M3_VALUES[c]) for c in range(256) if not math.isnan(oracle.E4M3_VALUES[c])]
    for yi, gi in zip(y[::7], got[::7]):
        a = float(yi)
        if abs(a) >= 448:
            assert gi == (0xFE if a < 0 else 0x7E)
            continue
        best = min(abs(val - a) for _, val in finite)
        cands = [c for c, val in finite if abs(val - a) == best and (val != 0 or math.copysign(1, a) == math.copysign(1, val))]
        if len(cands) > 1:
            cands = [c for c in cands if c % 2 == 0]
        assert gi in cands, (a, gi, cands)


def test_ties_go_to_the_even_code():
    v = oracle.E4M3_VALUES
    for c in list(range(0x00, 0x7D)) + list(range(0x80, 0xFD)):
        mid = np.float32((v[c] + v[c + 1]) / 2)
        if float(mid) != (v[c] + v[c + 1]) / 2:
            continue
        want = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_round(np.array([mid]))[0] == want, hex(c)


def test_quantize_scales_in_float32():
    # bf16(0.3) = 0.30078125; / 2 = 0.150390625, nearest E4M3 value 0.15625; 1000 / 2 saturates
    x = synth.to_storage(np.array([1.0, -3.0, 0.3, 1000.0], np.float32), "bf16")
    codes = oracle.quantize(x, "bf16", 2.0)
    assert list(oracle.e4m3_value(codes)) == [0.5, -1.5, 0.15625, 448.0]


def test_fp8_decode_step_is_attention_over_dequantized_values():
    case = synth.DecodeCase("f", 3, 8, 2, 16, "bf16", 1, 40, True, seed=31)
    inp = synth.fp8_decode_inputs(case)
    cache = oracle.PagedCache(inp["k_pool"], inp["v_pool"], inp["block_table"])
    O, L = oracle.decode_step_fp8(cache, inp["q"], inp["k_new"], inp["v_new"], inp["lens"], case.sm_scale, "bf16",
                                  0.5, 2.0)
    for b in range(case.B):
        n = int(inp["lens"][b]) + 1
        Kc, Vc = cache.gather(b, n)
        K = oracle.e4m3_value(Kc)[None] * 0.5
        V = oracle.e4m3_value(Vc)[None] * 2.0
        q = oracle.decode_bits(inp["q"][b], "bf16")[None, :, None, :]
        Oo, Lo = oracle.one_shot(q, K, V, case.sm_scale)
        assert np.max(np.abs(O[b] - Oo[0, :, 0])) <= 1e-12 and np.max(np.abs(L[b] - Lo[0, :, 0])) <= 1e-12
        # the new token's codes are the quantized new rows
        assert np.array_equal(Kc[:, -1], oracle.quantize(inp["k_new"][b, :, 0], "bf16", 0.5))
