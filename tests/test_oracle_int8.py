"""Pins of the int8 KV-cache oracle (per-channel scales): hand values, rounding
by brute force, ties, saturation, channel/head selection, decode over the
dequantized cache."""
import numpy as np
import pytest

import oracle
import synth


def _bits(vals, dtype="bf16"):
    return synth.to_storage(np.asarray(vals, np.float32), dtype)


def test_hand_values():
    # bf16(0.3) = 0.30078125; / 0.25 = 1.203125 -> 1
    x = _bits([1.0, -3.0, 0.3, 1000.0, -1000.0, 0.0]).reshape(1, 1, 6)
    s = np.full((1, 6), 0.25, np.float32)
    assert oracle.quantize_int8(x, "bf16", s).ravel().tolist() == [4, -12, 1, 127, -127, 0]


def test_ties_to_even_and_specials():
    x = np.array([2.5, 3.5, -2.5, -0.5, 0.5, 126.5, np.nan, np.inf, -np.inf], np.float32).reshape(1, 1, 9)
    s = np.ones((1, 9), np.float32)
    assert oracle.quantize_int8(x, "f32", s).ravel().tolist() == [2, 4, -2, 0, 0, 126, 0, 127, -127]


def test_rounding_against_brute_force():
    r = np.random.Generator(np.random.SFC64(9))
    n = 4000
    x = (r.standard_normal(n) * np.exp2(r.uniform(-8, 4, n))).astype(np.float32)
    s = np.exp2(r.uniform(-9, 0, n)).astype(np.float32)
    got = np.array([oracle.quantize_int8(x[i:i + 1].reshape(1, 1, 1), "f32", s[i:i + 1].reshape(1, 1))[0, 0, 0]
                    for i in range(0, n, 5)])
    for j, i in enumerate(range(0, n, 5)):
        y = float(np.float32(x[i]) / np.float32(s[i]))  # the float32 quotient
        best = min(range(-127, 128), key=lambda k: (abs(k - y), k % 2))  # nearest, ties to even
        assert got[j] == best, (x[i], s[i], y, got[j], best)


def test_scale_is_per_head_and_channel():
    H, n, d = 2, 3, 4
    s = np.array([[1, 2, 4, 8], [16, 32, 64, 128]], np.float32) / 128
    x = _bits(np.ones((H, n, d)), "f16")
    codes = oracle.quantize_int8(x, "f16", s)
    assert codes[0, 0].tolist() == [127, 64, 32, 16] and codes[1, 2].tolist() == [8, 4, 2, 1]
    back = oracle.dequantize_int8(codes, s)
    assert back[1, 1].tolist() == [8 * 16 / 128, 4 * 32 / 128, 2 * 64 / 128, 1.0]


def test_int8_decode_step_is_attention_over_dequantized_values():
    case = synth.DecodeCase("i", 3, 8, 2, 16, "bf16", 1, 40, True, seed=33)
    inp = synth.int8_decode_inputs(case)
    cache = oracle.PagedCache(inp["k_pool"], inp["v_pool"], inp["block_table"])
    O, L = oracle.decode_step_int8(cache, inp["q"], inp["k_new"], inp["v_new"], inp["lens"], case.sm_scale, "bf16",
                                   inp["k_scales"], inp["v_scales"])
    for b in range(case.B):
        n = int(inp["lens"][b]) + 1
        Kc, Vc = cache.gather(b, n)
        K = Kc.astype(np.float64) * inp["k_scales"].astype(np.float64)[:, None, :]
        V = Vc.astype(np.float64) * inp["v_scales"].astype(np.float64)[:, None, :]
        q = oracle.decode_bits(inp["q"][b], "bf16")[None, :, None, :]
        Oo, Lo = oracle.one_shot(q, K[None], V[None], case.sm_scale)
        assert np.max(np.abs(O[b] - Oo[0, :, 0])) <= 1e-12 and np.max(np.abs(L[b] - Lo[0, :, 0])) <= 1e-12
        # the new token's codes are the quantized new rows, channel by channel
        kn = oracle.decode_bits(inp["k_new"][b, :, 0], "bf16")
        want = np.clip(np.rint(kn.astype(np.float32) / inp["k_scales"]), -127, 127)
        assert np.array_equal(Kc[:, -1], want.astype(np.int8))


def test_int8_inputs_recipe():
    case = synth.DecodeCase("i", 4, 8, 2, 64, "bf16", 1, 100, True, seed=34)
    inp = synth.int8_decode_inputs(case)
    assert inp["k_pool"].dtype == np.int8 and inp["k_scales"].shape == (2, 64)
    assert inp["k_pool"].min() >= -127 and inp["v_pool"].min() >= -127
    outliers = inp["k_scales"] >= 2.0 ** -6
    assert outliers.sum(axis=1).tolist() == [4, 4]


def test_int4_packing_by_hand():
    codes = np.array([[1, -1, 7, -7, 0, -8, 3, 4]], np.int8)
    packed = oracle.pack_int4(codes)
    # element 2i in the low nibble, 2i + 1 in the high nibble, 4-bit two's complement
    assert packed.tolist() == [[0xF1, 0x97, 0x80, 0x43]]
    assert np.array_equal(oracle.unpack_int4(packed), codes)
    every = np.arange(256, dtype=np.uint8).reshape(1, 256)
    assert np.array_equal(oracle.pack_int4(oracle.unpack_int4(every)), every)


def test_int4_v_pool_order_by_hand():
    # positions worked out from the layout: run 16 (t // 4) + c % 16 of d / 8 bytes,
    # byte 4 ((c // 16) // 2) + (0, 2, 1, 3).index(t % 4), nibble (c // 16) % 2
    assert oracle.int4_v_position(0, 0, 128) == (0, 0)
    assert oracle.int4_v_position(5, 37, 128) == (21 * 16 + 4 + 2, 0)
    assert oracle.int4_v_position(14, 127, 128) == (63 * 16 + 12 + 1, 1)
    assert oracle.int4_v_position(3, 16, 128) == (3, 1)
    assert oracle.int4_v_position(9, 50, 64) == (34 * 8 + 4 + 2, 1)
    # one code placed through the row packing lands there, and nowhere else
    for t, c, d in ((5, 37, 128), (14, 127, 128), (9, 50, 64)):
        codes = np.zeros((16, d), np.int8)
        codes[t, c] = -3
        pool = oracle.int4_v_to_pool(oracle.pack_int4(codes)).ravel()
        off, hi = oracle.int4_v_position(t, c, d)
        want = np.zeros(8 * d, np.uint8)
        want[off] = 0xD << (4 * hi)  # -3 as a 4-bit two's complement nibble
        assert np.array_equal(pool, want)


def test_int4_v_pool_order_is_one_token_per_byte_and_a_permutation():
    for d in (64, 128):
        seen = {}
        for t in range(16):
            for c in range(d):
                off, hi = oracle.int4_v_position(t, c, d)
                assert 0 <= off < 8 * d and (off, hi) not in seen
                seen[(off, hi)] = (t, c)
        assert len(seen) == 16 * d
    with pytest.raises(ValueError):
        oracle.int4_v_position(0, 0, 16)
        for off in range(8 * d):  # a byte holds one token, channels c and c + 16
            (t0, c0), (t1, c1) = seen[(off, 0)], seen[(off, 1)]
            assert t0 == t1 and c1 == c0 + 16
    rng = np.random.default_rng(3)
    x = rng.integers(0, 256, size=(3, 2, 16, 32), dtype=np.uint8)
    assert np.array_equal(oracle.int4_v_to_pool(oracle.int4_v_from_pool(x)), x)
    assert np.array_equal(oracle.int4_v_from_pool(oracle.int4_v_to_pool(x)), x)


def test_int4_quantize_clamps_to_seven():
    x = np.array([6.4, 6.5, 7.5, 100.0, -7.5, -100.0, 2.5, np.nan], np.float32).reshape(1, 1, 8)
    s = np.ones((1, 8), np.float32)
    assert oracle.quantize_int4(x, "f32", s).ravel().tolist() == [6, 6, 7, 7, -7, -7, 2, 0]


def test_int4_decode_step_is_attention_over_dequantized_values():
    case = synth.DecodeCase("i4", 3, 8, 2, 32, "bf16", 1, 40, True, seed=35)
    inp = synth.int4_decode_inputs(case)
    assert inp["k_pool"].shape[-1] == 16
    cache = oracle.PagedCache(inp["k_pool"], inp["v_pool"], inp["block_table"])
    O, L = oracle.decode_step_int4(cache, inp["q"], inp["k_new"], inp["v_new"], inp["lens"], case.sm_scale, "bf16",
                                   inp["k_scales"], inp["v_scales"])
    rows = oracle.PagedCache(cache.k, oracle.int4_v_from_pool(cache.v), inp["block_table"])
    for b in range(case.B):
        n = int(inp["lens"][b]) + 1
        Kc, Vc = rows.gather(b, n)
        # nibbles decoded one by one, apart from unpack_int4
        def val(byte_arr, scales):
            out = np.empty(byte_arr.shape[:-1] + (2 * byte_arr.shape[-1],))
            for idx in np.ndindex(byte_arr.shape):
                byte = int(byte_arr[idx])
                lo, hi = byte & 15, byte >> 4
                out[idx[:-1] + (2 * idx[-1],)] = lo - 16 if lo >= 8 else lo
                out[idx[:-1] + (2 * idx[-1] + 1,)] = hi - 16 if hi >= 8 else hi
            return out * scales.astype(np.float64)[:, None, :]
        K, V = val(Kc, inp["k_scales"]), val(Vc, inp["v_scales"])
        q = oracle.decode_bits(inp["q"][b], "bf16")[None, :, None, :]
        Oo, Lo = oracle.one_shot(q, K[None], V[None], case.sm_scale)
        assert np.max(np.abs(O[b] - Oo[0, :, 0])) <= 1e-12 and np.max(np.abs(L[b] - Lo[0, :, 0])) <= 1e-12
