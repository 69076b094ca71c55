"""Pins of the cache models: byte-exact append images and paged == contiguous."""
import numpy as np
import pytest

import oracle
import synth
from synth import DecodeCase


def _case(paged, B=3, lo=1, hi=40, n_new=1, dtype="bf16"):
    return DecodeCase("t", B, 4, 2, 8, dtype, lo, hi, paged, seed=5, n_new=n_new)


def test_contig_append_image_bytes():
    case = _case(False, n_new=3)
    inp = synth.decode_inputs(case)
    cache = oracle.ContigCache(inp["k_cache"], inp["v_cache"])
    before_k, before_v = cache.k.copy(), cache.v.copy()
    cache.append(inp["k_new"], inp["v_new"], inp["lens"])
    # expected image written by hand: only the n_new slots after each length change
    ek, ev = before_k.copy(), before_v.copy()
    for b, L in enumerate(inp["lens"]):
        ek[b, :, L:L + 3] = inp["k_new"][b]
        ev[b, :, L:L + 3] = inp["v_new"][b]
    assert cache.k.tobytes() == ek.tobytes() and cache.v.tobytes() == ev.tobytes()
    # sentinels beyond the new length stay untouched
    sk = synth.storage_fill((1,), synth.SENTINEL_V, "bf16")[0]
    for b, L in enumerate(inp["lens"]):
        assert np.all(cache.v[b, :, L + 3:] == sk)


def test_contig_append_overflow_raises():
    case = _case(False)
    inp = synth.decode_inputs(case)
    cache = oracle.ContigCache(inp["k_cache"], inp["v_cache"])
    bad = inp["lens"].copy()
    bad[0] = case.max_len
    with pytest.raises(IndexError):
        cache.append(inp["k_new"], inp["v_new"], bad)


@pytest.mark.parametrize("n_new", [1, 5, 17])
def test_paged_gather_equals_contiguous(n_new):
    """Same draws, two layouts: gathering the pool through the table is the contiguous cache."""
    pc, cc = _case(True, n_new=n_new), _case(False, n_new=n_new)
    pin, cin = synth.decode_inputs(pc), synth.decode_inputs(cc)
    assert np.array_equal(pin["lens"], cin["lens"])
    paged = oracle.PagedCache(pin["k_pool"], pin["v_pool"], pin["block_table"])
    contig = oracle.ContigCache(cin["k_cache"], cin["v_cache"])
    paged.append(pin["k_new"], pin["v_new"], pin["lens"])
    contig.append(cin["k_new"], cin["v_new"], cin["lens"])
    for b, L in enumerate(pin["lens"] + n_new):
        kp, vp = paged.gather(b, int(L))
        kc, vc = contig.view(b, int(L))
        assert kp.tobytes() == np.ascontiguousarray(kc).tobytes()
        assert vp.tobytes() == np.ascontiguousarray(vc).tobytes()


def test_identity_table_is_reshape():
    B, H, nb, d = 2, 3, 4, 5
    pool = np.arange(B * nb * H * 16 * d, dtype=np.float32).reshape(B * nb, H, 16, d)
    table = np.arange(B * nb, dtype=np.int32).reshape(B, nb)
    pc = oracle.PagedCache(pool, pool + 0.5, table)
    for b in range(B):
        K, _ = pc.gather(b, nb * 16)
        expect = pool[b * nb:(b + 1) * nb].transpose(1, 0, 2, 3).reshape(H, nb * 16, d)
        assert np.array_equal(K, expect)


def test_paged_rejects_unassigned_block():
    pool = np.zeros((2, 1, 16, 2), np.float32)
    table = np.array([[0, -1]], np.int32)
    pc = oracle.PagedCache(pool, pool, table)
    with pytest.raises(IndexError):
        pc.append(np.ones((1, 1, 1, 2), np.float32), np.ones((1, 1, 1, 2), np.float32), [16])


def test_list_cache_roundtrip():
    lc = oracle.ListCache(2, 3)
    lc.append(1, 2, [1.0, 2.0], [3.0, 4.0])
    lc.append(1, 2, [5.0, 6.0], [7.0, 8.0])
    K, V = lc.read(1, 2)
    assert [list(x) for x in K] == [[1.0, 2.0], [5.0, 6.0]]
    assert lc.read(0, 0) == ([], [])


def test_generated_table_is_a_permutation():
    case = _case(True, B=6, lo=0, hi=70)
    inp = synth.decode_inputs(case)
    t = inp["block_table"]
    used = t[t >= 0]
    assert sorted(used.tolist()) == list(range(inp["k_pool"].shape[0]))
    for b, L in enumerate(inp["lens"] + 1):
        assert np.all(t[b, :-(-int(L) // 16)] >= 0) and np.all(t[b, -(-int(L) // 16):] == -1)
