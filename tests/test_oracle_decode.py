"""Pins of the decoders: cached == naive, operation counts, decode and chunk steps == causal prefill rows."""
import json
import os

import numpy as np

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _stream(seed, n, H_q, H_kv, d):
    r = np.random.Generator(np.random.SFC64(seed))
    qs = [r.standard_normal((H_q, d)) for _ in range(n)]
    ks = [r.standard_normal((H_kv, d)) for _ in range(n)]
    vs = [r.standard_normal((H_kv, d)) for _ in range(n)]
    return qs, ks, vs


def test_cached_equals_naive_and_counts():
    golden = json.load(open(os.path.join(GOLDEN, "op_counts.json")))
    for c in golden["cases"]:
        n = c["n"]
        qs, ks, vs = _stream(1, n, 4, 2, 3)
        Oc, nc = oracle.cached_decode(qs, ks, vs, 0.5)
        On, nn = oracle.naive_decode(qs, ks, vs, 0.5)
        assert np.array_equal(Oc, On)  # same routine on the same data: bit-identical
        assert (nn, nc) == (c["naive"], c["cached"]), c["cite"]
    for n in (1, 2, 7, 31):
        qs, ks, vs = _stream(n, n, 2, 1, 2)
        assert oracle.naive_decode(qs, ks, vs, 1.0)[1] == n * (n + 1) // 2
        assert oracle.cached_decode(qs, ks, vs, 1.0)[1] == n


def test_decode_step_equals_causal_prefill_row():
    """Step t of incremental decoding is row t of causal prefill over the whole sequence."""
    n, H_q, H_kv, d = 12, 4, 2, 5
    qs, ks, vs = _stream(3, n, H_q, H_kv, d)
    Oc, _ = oracle.cached_decode(qs, ks, vs, 0.4)
    Q = np.stack(qs, axis=1)[None]  # [1, H_q, n, d]
    K = np.stack(ks, axis=1)[None]
    V = np.stack(vs, axis=1)[None]
    Op, _ = oracle.one_shot(Q, K, V, 0.4, causal=True)
    for t in range(n):
        assert np.max(np.abs(Oc[t] - Op[0, :, t])) <= 1e-12


def test_decode_step_contig_and_paged_agree():
    for n_new in (1, 3):
        common = dict(B=4, H_q=8, H_kv=2, d=16, dtype="bf16", len_lo=1, len_hi=50, seed=9, n_new=n_new)
        cc = synth.DecodeCase("c", paged=False, **common)
        pc = synth.DecodeCase("p", paged=True, **common)
        ci, pi = synth.decode_inputs(cc), synth.decode_inputs(pc)
        Oc, Lc = oracle.decode_step(oracle.ContigCache(ci["k_cache"], ci["v_cache"]), ci["q"],
                                    ci["k_new"], ci["v_new"], ci["lens"], cc.sm_scale, "bf16")
        Op, Lp = oracle.decode_step(oracle.PagedCache(pi["k_pool"], pi["v_pool"], pi["block_table"]),
                                    pi["q"], pi["k_new"], pi["v_new"], pi["lens"], pc.sm_scale, "bf16")
        assert np.array_equal(Oc, Op) and np.array_equal(Lc, Lp)


def test_decode_step_against_one_shot():
    case = synth.DecodeCase("c", 3, 4, 2, 8, "f32", 1, 20, False, seed=11)
    inp = synth.decode_inputs(case)
    O, L = oracle.decode_step(oracle.ContigCache(inp["k_cache"], inp["v_cache"]), inp["q"],
                              inp["k_new"], inp["v_new"], inp["lens"], case.sm_scale, "f32")
    for b in range(case.B):
        n = int(inp["lens"][b])
        K = np.concatenate([inp["k_cache"][b, :, :n], inp["k_new"][b]], axis=1).astype(np.float64)
        V = np.concatenate([inp["v_cache"][b, :, :n], inp["v_new"][b]], axis=1).astype(np.float64)
        q = inp["q"][b].astype(np.float64)[None, :, None, :]
        Oo, Lo = oracle.one_shot(q, K[None], V[None], case.sm_scale)
        assert np.max(np.abs(O[b] - Oo[0, :, 0])) <= 1e-12
        assert np.max(np.abs(L[b] - Lo[0, :, 0])) <= 1e-12


def _chunk_case(seed, Ls, n, H_q, H_kv, d):
    """Whole sequences (float32 storage) and the caches holding their first L_b tokens."""
    r = np.random.Generator(np.random.SFC64(seed))
    B = len(Ls)
    full = [{x: r.standard_normal((H, Lb + n, d)).astype(np.float32)
             for x, H in (("q", H_q), ("k", H_kv), ("v", H_kv))} for Lb in Ls]
    cap = max(Ls) + n
    kc = np.zeros((B, H_kv, cap, d), np.float32)
    vc = np.zeros((B, H_kv, cap, d), np.float32)
    for b, Lb in enumerate(Ls):
        kc[b, :, :Lb] = full[b]["k"][:, :Lb]
        vc[b, :, :Lb] = full[b]["v"][:, :Lb]
    q = np.stack([f["q"][:, Lb:] for f, Lb in zip(full, Ls)])
    kn = np.stack([f["k"][:, Lb:] for f, Lb in zip(full, Ls)])
    vn = np.stack([f["v"][:, Lb:] for f, Lb in zip(full, Ls)])
    return full, oracle.ContigCache(kc, vc), q, kn, vn, np.array(Ls, np.int32)


def test_chunk_step_equals_causal_prefill_rows():
    """A chunk's queries are the last n rows of causal prefill over the whole sequence."""
    Ls, n, H_q, H_kv, d = [0, 5, 17], 6, 4, 2, 8
    full, cache, q, kn, vn, lens = _chunk_case(21, Ls, n, H_q, H_kv, d)
    O, L = oracle.chunk_step(cache, q, kn, vn, lens, 0.3, "f32")
    for b, Lb in enumerate(Ls):
        f = {x: full[b][x].astype(np.float64)[None] for x in ("q", "k", "v")}
        Op, Lp = oracle.one_shot(f["q"], f["k"], f["v"], 0.3, causal=True)
        assert np.max(np.abs(O[b] - Op[0, :, Lb:])) <= 1e-12
        assert np.max(np.abs(L[b] - Lp[0, :, Lb:])) <= 1e-12


def test_chunk_step_non_causal_sees_every_key():
    Ls, n, H_q, H_kv, d = [3, 9], 4, 2, 1, 5
    full, cache, q, kn, vn, lens = _chunk_case(22, Ls, n, H_q, H_kv, d)
    O, L = oracle.chunk_step(cache, q, kn, vn, lens, 0.5, "f32", causal=False)
    for b, Lb in enumerate(Ls):
        f = {x: full[b][x].astype(np.float64)[None] for x in ("q", "k", "v")}
        Oo, Lo = oracle.one_shot(f["q"][:, :, Lb:], f["k"], f["v"], 0.5, causal=False)
        assert np.max(np.abs(O[b] - Oo[0])) <= 1e-12 and np.max(np.abs(L[b] - Lo[0])) <= 1e-12


def test_chunk_step_of_one_token_is_a_decode_step():
    case = synth.DecodeCase("c", 3, 4, 2, 8, "bf16", 1, 40, True, seed=23)
    inp = synth.decode_inputs(case)
    mk = lambda: oracle.PagedCache(inp["k_pool"].copy(), inp["v_pool"].copy(), inp["block_table"])
    Od, Ld = oracle.decode_step(mk(), inp["q"], inp["k_new"], inp["v_new"], inp["lens"], case.sm_scale, "bf16")
    Oc, Lc = oracle.chunk_step(mk(), inp["q"][:, :, None, :], inp["k_new"], inp["v_new"], inp["lens"],
                               case.sm_scale, "bf16")
    assert np.array_equal(Oc[:, :, 0], Od) and np.array_equal(Lc[:, :, 0], Ld)


def test_chunk_step_contig_and_paged_agree():
    common = dict(B=3, H_q=4, H_kv=2, d=16, dtype="f16", len_lo=0, len_hi=40, seed=24, n_new=7)
    cc = synth.DecodeCase("c", paged=False, **common)
    pc = synth.DecodeCase("p", paged=True, **common)
    ci, pi = synth.chunk_inputs(cc), synth.chunk_inputs(pc)
    Oc, Lc = oracle.chunk_step(oracle.ContigCache(ci["k_cache"], ci["v_cache"]), ci["q"],
                               ci["k_new"], ci["v_new"], ci["lens"], cc.sm_scale, "f16")
    Op, Lp = oracle.chunk_step(oracle.PagedCache(pi["k_pool"], pi["v_pool"], pi["block_table"]),
                               pi["q"], pi["k_new"], pi["v_new"], pi["lens"], pc.sm_scale, "f16")
    assert np.array_equal(Oc, Op) and np.array_equal(Lc, Lp)
