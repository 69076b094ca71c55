"""GPU parity of kv_append (bit-exact) and attn_decode / attn_decode_paged (oracle tolerance)."""
import numpy as np
import pytest

import oracle
import synth
from helpers import (assert_close, assert_lse_close, assert_stored_output, bits_of, extreme_queries, to_dev,
                     to_dev_i32, values_of)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_flashattention_attn_amd as k
    k.lib()
    assert k.attn_device_error_flags() == 0
    return k


def run_step(K, case, lens=None, heads=None, inp=None):
    """One append + attend step on the GPU and in the oracle; returns GPU (O, lse).

    16-bit outputs are checked with the stored-output rule: the same call with
    the fp32 output meets the bar, and the stored output is its
    round-to-nearest-even."""
    print(f"[decode] {case}", flush=True)
    inp = synth.decode_inputs(case, lens=lens) if inp is None else inp
    dt = case.dtype
    lens_d = to_dev_i32(inp["lens"])
    seq_d = to_dev_i32(inp["lens"] + case.n_new)
    q, kn, vn = to_dev(inp["q"], dt), to_dev(inp["k_new"], dt), to_dev(inp["v_new"], dt)
    if case.paged:
        kc, vc = to_dev(inp["k_pool"], dt), to_dev(inp["v_pool"], dt)
        table = to_dev_i32(inp["block_table"])
        K.kv_append(kc, vc, kn, vn, lens_d, table)
        o, lse = K.attn_decode_paged(q, kc, vc, table, seq_d, scale=case.sm_scale, return_lse=True)
        o32 = K.attn_decode_paged(q, kc, vc, table, seq_d, scale=case.sm_scale, out_fp32=True)
        ocache = oracle.PagedCache(inp["k_pool"], inp["v_pool"], inp["block_table"])
    else:
        kc, vc = to_dev(inp["k_cache"], dt), to_dev(inp["v_cache"], dt)
        K.kv_append(kc, vc, kn, vn, lens_d)
        o, lse = K.attn_decode(q, kc, vc, seq_d, scale=case.sm_scale, return_lse=True)
        o32 = K.attn_decode(q, kc, vc, seq_d, scale=case.sm_scale, out_fp32=True)
        ocache = oracle.ContigCache(inp["k_cache"], inp["v_cache"])
    torch.cuda.synchronize()
    assert K.attn_device_error_flags() == 0
    Oref, Lref = oracle.decode_step(ocache, inp["q"], inp["k_new"], inp["v_new"], inp["lens"],
                                    case.sm_scale, dt, heads=heads)
    # the append image, byte for byte (whole buffers, untouched sentinels included)
    assert bits_of(kc).tobytes() == ocache.k.tobytes(), "K cache image differs"
    assert bits_of(vc).tobytes() == ocache.v.tobytes(), "V cache image differs"
    got_o, got_o32, got_l = o, o32, lse.cpu().numpy().astype(np.float64)
    if heads is not None:
        idx = tuple(np.array(heads).T)
        got_o, got_o32, Oref, got_l, Lref = got_o[idx], got_o32[idx], Oref[idx], got_l[idx], Lref[idx]
    if dt == "f32":
        assert_close(values_of(got_o), Oref, dt)
        assert torch.equal(got_o, got_o32)
    else:
        assert_stored_output(got_o, got_o32, Oref, dt)
    assert_lse_close(got_l, Lref, dt)
    return o, lse


def case(paged, B, H_q, H_kv, d, dtype, lo, hi, seed, n_new=1):
    return synth.DecodeCase("sweep", B, H_q, H_kv, d, dtype, lo, hi, paged, seed, n_new=n_new)


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_chunk_boundaries(K, paged, dtype, d):
    """Cache lengths around block (16), step (32) and chunk (256/512) boundaries."""
    lens = np.array([0, 14, 15, 16, 30, 31, 255, 511, 512, 1023, 1500], dtype=np.int32)
    run_step(K, case(paged, len(lens), 8, 2, d, dtype, 0, 1600, 10 + d), lens=lens)


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16, 32])
def test_decode_gqa_groups(K, paged, G):
    run_step(K, case(paged, 3, 2 * G, 2, 128, "bf16", 1, 700, 20 + G))


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("d", [16, 32, 256])
def test_decode_plain_path(K, paged, dtype, d):
    run_step(K, case(paged, 3, 4, 2, d, dtype, 1, 600, 30 + d))


@pytest.mark.parametrize("paged", [False, True])
def test_many_short_sequences(K, paged):
    """300 sequences of 0 .. 200 cached tokens: most waves cross many segment
    boundaries (query reload, state reset and a piece write at each)."""
    o1, _ = run_step(K, case(paged, 300, 32, 8, 128, "bf16", 0, 200, 95))
    o2, _ = run_step(K, case(paged, 300, 32, 8, 128, "bf16", 0, 200, 95))
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("paged", [False, True])
def test_one_long_sequence_many_pieces(K, paged):
    """One sequence of 40,000 tokens and one KV head: the whole grid shares one
    segment, cut into ~157 pieces, so the merge combines more than 64 partials."""
    run_step(K, case(paged, 1, 8, 1, 128, "bf16", 39999, 39999, 90))


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("n_new", [3, 17])
def test_multi_token_append(K, paged, n_new):
    run_step(K, case(paged, 4, 8, 4, 128, "bf16", 0, 90, 40 + n_new, n_new=n_new))


# 16-bit patterns written into cache slots that hold no token
NONFINITE = {"bf16": (0x7FC0, 0x7F80, 0xFF80), "f16": (0x7E00, 0x7C00, 0xFC00)}  # NaN, +inf, -inf


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_ignores_nonfinite_slots_past_the_length(K, paged, dtype, d):
    """Slots at or past a sequence's length may hold anything: here K holds NaN
    and V cycles through NaN, +inf and -inf.  None of it may reach O or lse (a
    weight of 0 times a NaN or an infinity is not 0, so such rows must never be
    multiplied at all)."""
    lens = np.array([0, 1, 14, 15, 17, 31, 100, 255, 256], dtype=np.int32)
    c = case(paged, len(lens), 8, 2, d, dtype, 0, 300, 200 + d)
    inp = synth.decode_inputs(c, lens=lens)
    nan, pinf, ninf = NONFINITE[dtype]
    after = lens + c.n_new  # tokens held once the append has run
    if paged:
        kp, vp, table = inp["k_pool"], inp["v_pool"], inp["block_table"]
        held = np.zeros(kp.shape[0] * 16, dtype=bool)
        for b in range(c.B):
            for t in range(int(after[b])):
                held[table[b, t // 16] * 16 + t % 16] = True
        empty = ~held.reshape(kp.shape[0], 1, 16, 1).repeat(c.H_kv, 1).repeat(d, 3)
        kk, vv = kp, vp
    else:
        kk, vv = inp["k_cache"], inp["v_cache"]
        empty = np.arange(kk.shape[2])[None, None, :, None] >= after[:, None, None, None]
        empty = np.broadcast_to(empty, kk.shape)
    pattern = np.array([nan, pinf, ninf], dtype=np.uint16)[np.arange(vv.size).reshape(vv.shape) % 3]
    kk[empty] = nan
    vv[empty] = pattern[empty]
    run_step(K, c, inp=inp)


def test_paged_identity_table_matches_contiguous(K):
    """Identity block table: the paged pool is a reshaped contiguous cache."""
    B, H_kv, H_q, d, nb = 2, 2, 8, 128, 6
    r = np.random.Generator(np.random.SFC64(50))
    pool_k = synth.to_storage(r.standard_normal((B * nb, H_kv, 16, d), dtype=np.float32), "bf16")
    pool_v = synth.to_storage(r.standard_normal((B * nb, H_kv, 16, d), dtype=np.float32), "bf16")
    qn = synth.to_storage(r.standard_normal((B, H_q, d), dtype=np.float32), "bf16")
    table = np.arange(B * nb, dtype=np.int32).reshape(B, nb)
    contig_k = pool_k.reshape(B, nb, H_kv, 16, d).transpose(0, 2, 1, 3, 4).reshape(B, H_kv, nb * 16, d)
    contig_v = pool_v.reshape(B, nb, H_kv, 16, d).transpose(0, 2, 1, 3, 4).reshape(B, H_kv, nb * 16, d)
    lens = np.array([nb * 16, 37], dtype=np.int32)
    q = to_dev(qn, "bf16")
    op = K.attn_decode_paged(q, to_dev(pool_k, "bf16"), to_dev(pool_v, "bf16"), to_dev_i32(table), to_dev_i32(lens))
    oc = K.attn_decode(q, to_dev(contig_k, "bf16"), to_dev(contig_v, "bf16"), to_dev_i32(lens))
    torch.cuda.synchronize()
    assert torch.equal(op.view(torch.int16), oc.view(torch.int16))


def test_decode_repeatable(K):
    """The same inputs give the same bits on every call (each call on fresh copies of the cache)."""
    B, H_kv, H_q, d, nb = 2, 2, 8, 128, 6
    r = np.random.Generator(np.random.SFC64(51))
    pool_k = synth.to_storage(r.standard_normal((B * nb, H_kv, 16, d), dtype=np.float32), "bf16")
    pool_v = synth.to_storage(r.standard_normal((B * nb, H_kv, 16, d), dtype=np.float32), "bf16")
    qn = synth.to_storage(r.standard_normal((B, H_q, d), dtype=np.float32), "bf16")
    table = np.arange(B * nb, dtype=np.int32).reshape(B, nb)
    contig_k = np.ascontiguousarray(pool_k.reshape(B, nb, H_kv, 16, d).transpose(0, 2, 1, 3, 4).reshape(B, H_kv, nb * 16, d))
    contig_v = np.ascontiguousarray(pool_v.reshape(B, nb, H_kv, 16, d).transpose(0, 2, 1, 3, 4).reshape(B, H_kv, nb * 16, d))
    lens = to_dev_i32(np.array([nb * 16, 37], dtype=np.int32))
    q = to_dev(qn, "bf16")
    outs = []
    for _ in range(8):
        oc = K.attn_decode(q, to_dev(contig_k, "bf16"), to_dev(contig_v, "bf16"), lens)
        op = K.attn_decode_paged(q, to_dev(pool_k, "bf16"), to_dev(pool_v, "bf16"), to_dev_i32(table), lens)
        torch.cuda.synchronize()
        outs.append((bits_of(oc), bits_of(op)))
    for oc, op in outs:
        assert np.array_equal(oc, outs[0][0]) and np.array_equal(op, outs[0][0])


@pytest.mark.parametrize("d", [64, 128])
def test_contiguous_capacity_not_multiple_of_16(K, d):
    """A contiguous cache of 37 rows: the last 16-token stage reaches past the capacity
    (those rows are read from the last row and masked)."""
    B, H_kv, H_q, cap = 3, 2, 8, 37
    r = np.random.Generator(np.random.SFC64(70 + d))
    kc = synth.to_storage(r.standard_normal((B, H_kv, cap, d), dtype=np.float32), "bf16")
    vc = synth.to_storage(r.standard_normal((B, H_kv, cap, d), dtype=np.float32), "bf16")
    qn = synth.to_storage(r.standard_normal((B, H_q, d), dtype=np.float32), "bf16")
    lens = np.array([37, 33, 16], dtype=np.int32)
    print(f"[decode] contiguous capacity {cap}, d={d}, lens={lens.tolist()}", flush=True)
    o, lse = K.attn_decode(to_dev(qn, "bf16"), to_dev(kc, "bf16"), to_dev(vc, "bf16"), to_dev_i32(lens),
                           return_lse=True)
    torch.cuda.synchronize()
    assert K.attn_device_error_flags() == 0
    Q, Kk, V = (oracle.decode_bits(x, "bf16") for x in (qn, kc, vc))
    Oref = np.zeros((B, H_q, d))
    Lref = np.zeros((B, H_q))
    for b in range(B):
        L = int(lens[b])
        ob, lb = oracle.one_shot(Q[b:b + 1, :, None, :], Kk[b:b + 1, :, :L], V[b:b + 1, :, :L], 1 / np.sqrt(d))
        Oref[b], Lref[b] = ob[0, :, 0], lb[0, :, 0]
    assert_close(values_of(o), Oref, "bf16")
    assert_lse_close(lse.cpu().numpy().astype(np.float64), Lref, "bf16")


def test_decode_zero_length_gives_zero(K):
    lens = np.array([0, 5], dtype=np.int32)
    c = case(False, 2, 4, 2, 128, "bf16", 0, 10, 60)
    inp = synth.decode_inputs(c, lens=lens)
    q = to_dev(inp["q"], "bf16")
    o, lse = K.attn_decode(q, to_dev(inp["k_cache"], "bf16"), to_dev(inp["v_cache"], "bf16"),
                           to_dev_i32(np.array([0, 5], np.int32)), return_lse=True)
    torch.cuda.synchronize()
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))
    assert torch.all(torch.isfinite(lse[1]))


def test_bad_lengths_and_blocks_raise_device_flags(K):
    """Out-of-range lengths and block ids are clamped/skipped and reported, never faulted on."""
    c = case(True, 2, 4, 2, 128, "bf16", 20, 40, 70)
    inp = synth.decode_inputs(c)
    dt = "bf16"
    kc, vc = to_dev(inp["k_pool"], dt), to_dev(inp["v_pool"], dt)
    table = inp["block_table"].copy()
    table[0, 1] = kc.shape[0] + 5          # out-of-range block id
    table_d = to_dev_i32(table)
    K.kv_append(kc, vc, to_dev(inp["k_new"], dt), to_dev(inp["v_new"], dt),
                to_dev_i32(np.array([20, 1000], np.int32)), table_d)  # seq 0 writes into the bad block
    assert K.attn_device_error_flags() & 3 != 0
    seq = to_dev_i32(np.array([40, 10 ** 6], np.int32))   # seq 1 beyond the table's capacity
    K.attn_decode_paged(to_dev(inp["q"], dt), kc, vc, table_d, seq)
    flags = K.attn_device_error_flags()
    assert flags & 1 and flags & 2
    # contiguous: length beyond max_len
    cc = case(False, 2, 4, 2, 128, "bf16", 5, 9, 71)
    ci = synth.decode_inputs(cc)
    K.attn_decode(to_dev(ci["q"], dt), to_dev(ci["k_cache"], dt), to_dev(ci["v_cache"], dt),
                  to_dev_i32(np.array([cc.max_len + 100, -3], np.int32)))
    flags = K.attn_device_error_flags()
    assert flags & 1 and flags & 4
    assert K.attn_device_error_flags() == 0   # cleared by the read


def test_decode_deterministic(K):
    c = case(True, 4, 16, 2, 128, "bf16", 100, 3000, 80)
    inp = synth.decode_inputs(c)
    dt = "bf16"
    args = (to_dev(inp["q"], dt), to_dev(inp["k_pool"], dt), to_dev(inp["v_pool"], dt),
            to_dev_i32(inp["block_table"]), to_dev_i32(inp["lens"]))
    o1, o2 = K.attn_decode_paged(*args), K.attn_decode_paged(*args)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_oracle_catches_a_corrupted_block_table(K):
    """Teeth: a table entry pointing at another sequence's block must break agreement.

    (Swapping two entries of one sequence would not: it permutes K and V rows
    together, which attention is invariant to.)
    """
    c = case(True, 2, 8, 2, 128, "bf16", 300, 400, 90)
    inp = synth.decode_inputs(c)
    dt = "bf16"
    table = inp["block_table"].copy()
    table[0, 2] = table[1, 5]
    seq = inp["lens"]
    o = K.attn_decode_paged(to_dev(inp["q"], dt), to_dev(inp["k_pool"], dt), to_dev(inp["v_pool"], dt),
                            to_dev_i32(table), to_dev_i32(seq), scale=c.sm_scale)
    torch.cuda.synchronize()
    pc = oracle.PagedCache(inp["k_pool"], inp["v_pool"], inp["block_table"])
    # attend over the first `seq` tokens without an append: reuse decode_step with n_new=0 rows
    empty = np.zeros((c.B, c.H_kv, 0, c.d), dtype=np.uint16)
    Oref, _ = oracle.decode_step(pc, inp["q"], empty, empty, seq, c.sm_scale, dt)
    err = np.abs(values_of(o)[0] - Oref[0]).max()
    assert err > 1e-2


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_decode_extreme_queries(K, paged, dtype):
    """Query heads that are all zero, one dominant channel over tiny ones, tiny,
    or large (logits near 60)."""
    c = case(paged, 4, 8, 2, 128, dtype, 1, 300, 330 + paged)
    inp = synth.decode_inputs(c)
    extreme_queries(inp, dtype)
    run_step(K, c, inp=inp)
