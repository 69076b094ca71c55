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


def _e4m3_by_formula(c):
    """Value of one E4M3 code from its bit fields (independent of the table)."""
    c = int(c)
    s, e, m = (c >> 7) & 1, (c >> 3) & 15, c & 7
    mag = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
    return -mag if s else mag


def test_fp8_prefill_is_brute_force_attention_over_dequantized_values():
    case = synth.PrefillCase("f8p", 1, 4, 2, 9, 8, "bf16", True, True, 41)
    inp = synth.fp8_prefill_inputs(case)
    qs, ks, vs, scale = 0.5, 0.25, 2.0, 0.3
    O, L = oracle.prefill_fp8(inp["q"], inp["k"], inp["v"], qs, ks, vs, scale, causal=True)
    deq = np.vectorize(_e4m3_by_formula)
    Q, K, V = deq(inp["q"]) * qs, deq(inp["k"]) * ks, deq(inp["v"]) * vs
    Ob, Lb = oracle.brute_attention(Q, K, V, scale, causal=True)
    assert np.max(np.abs(O - Ob)) <= 1e-12 and np.max(np.abs(L - Lb)) <= 1e-12


def test_fp8_prefill_scales_enter_as_stated():
    case = synth.PrefillCase("f8p", 1, 2, 1, 33, 16, "bf16", False, True, 42)
    inp = synth.fp8_prefill_inputs(case)
    O1, L1 = oracle.prefill_fp8(inp["q"], inp["k"], inp["v"], 1.0, 1.0, 1.0, 0.25, causal=False)
    # q_scale and k_scale multiply the logits like scale does; v_scale scales O and leaves lse
    O2, L2 = oracle.prefill_fp8(inp["q"], inp["k"], inp["v"], 2.0, 0.5, 4.0, 0.25, causal=False)
    O3, L3 = oracle.prefill_fp8(inp["q"], inp["k"], inp["v"], 2.0, 1.0, 1.0, 0.125, causal=False)
    assert np.allclose(O2, 4.0 * O1, atol=1e-12) and np.allclose(L2, L1, atol=1e-12)
    assert np.allclose(O3, O1, atol=1e-12) and np.allclose(L3, L1, atol=1e-12)
    rows = [(0, 1, 0), (0, 0, 32), (0, 1, 17)]
    Or, Lr = oracle.prefill_fp8(inp["q"], inp["k"], inp["v"], 1.0, 1.0, 1.0, 0.25, causal=False, rows=rows)
    for r, (b, h, i) in enumerate(rows):
        assert np.allclose(Or[r], O1[b, h, i], atol=1e-12) and abs(Lr[r] - L1[b, h, i]) <= 1e-12
