"""GPU parity of attn_prefill_paged (a chunk of new tokens against a paged cache) with the oracle."""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_close, assert_lse_close, bits_of, to_dev, to_dev_i32, values_of

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


def run_chunk(K, case, lens=None, causal=True, rows=None):
    """Paged append of the chunk, then attn_prefill_paged; compared with oracle.chunk_step."""
    print(f"[chunk] {case} causal={causal}", flush=True)
    inp = synth.chunk_inputs(case, lens=lens)
    dt = case.dtype
    lens_d = to_dev_i32(inp["lens"])
    q, kn, vn = to_dev(inp["q"], dt), to_dev(inp["k_new"], dt), to_dev(inp["v_new"], dt)
    kp, vp = to_dev(inp["k_pool"], dt), to_dev(inp["v_pool"], dt)
    table = to_dev_i32(inp["block_table"])
    K.kv_append(kp, vp, kn, vn, lens_d, table)
    o, lse = K.attn_prefill_paged(q, kp, vp, table, lens_d, causal=causal, scale=case.sm_scale, return_lse=True)
    torch.cuda.synchronize()
    assert K.attn_device_error_flags() == 0
    cache = oracle.PagedCache(inp["k_pool"], inp["v_pool"], inp["block_table"])
    Oref, Lref = oracle.chunk_step(cache, inp["q"], inp["k_new"], inp["v_new"], inp["lens"], case.sm_scale, dt,
                                   causal=causal, rows=rows)
    assert bits_of(kp).tobytes() == cache.k.tobytes(), "K pool image differs"
    assert bits_of(vp).tobytes() == cache.v.tobytes(), "V pool image differs"
    got_o, got_l = values_of(o), lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        idx = tuple(np.array(rows).T)
        got_o, Oref, got_l, Lref = got_o[idx], Oref[idx], got_l[idx], Lref[idx]
    assert_close(got_o, Oref, dt)
    assert_lse_close(got_l, Lref, dt)
    return o, lse


def case(B, H_q, H_kv, d, dtype, lo, hi, seed, n_new):
    return synth.DecodeCase("chunk", B, H_q, H_kv, d, dtype, lo, hi, True, seed, n_new=n_new)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
def test_chunk_prefix_lengths(K, d, dtype, causal):
    """Prefixes around block (16) and tile (64) boundaries, a ragged chunk of 37 tokens."""
    lens = np.array([0, 1, 15, 16, 17, 63, 64, 100, 255, 300], dtype=np.int32)
    run_chunk(K, case(len(lens), 8, 2, d, dtype, 0, 400, 50 + d, 37), lens=lens, causal=causal)


@pytest.mark.parametrize("n_new", [1, 16, 64, 129, 200])
def test_chunk_sizes(K, n_new):
    run_chunk(K, case(4, 4, 4, 128, "bf16", 0, 500, 60 + n_new, n_new))


@pytest.mark.parametrize("G", [1, 4, 8])
def test_chunk_gqa_groups(K, G):
    run_chunk(K, case(3, 2 * G, 2, 128, "bf16", 10, 700, 70 + G, 96))


def test_chunk_with_empty_prefix_is_causal_prefill(K):
    """Prefix 0: the chunk kernel and the contiguous prefill kernel see the same problem."""
    c = case(2, 4, 2, 128, "bf16", 0, 0, 80, 300)
    inp = synth.chunk_inputs(c, lens=np.zeros(2, np.int32))
    o_chunk, l_chunk = run_chunk(K, c, lens=np.zeros(2, np.int32))
    kcont = to_dev(inp["k_new"], "bf16")
    vcont = to_dev(inp["v_new"], "bf16")
    o_pre, l_pre = K.attn_prefill(to_dev(inp["q"], "bf16"), kcont, vcont, causal=True, scale=c.sm_scale,
                                  return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o_chunk, o_pre) and torch.equal(l_chunk, l_pre)


def test_chunk_workload_sampled_rows(K):
    """The 16 x 512-token chunk workload after prefixes of 0 .. 4096, on sampled rows."""
    c = synth.CHUNK_PAGED
    r = np.random.Generator(np.random.SFC64(77))
    rows = sorted({(int(b), int(h), int(t)) for b, h, t in zip(r.integers(0, c.B, 48), r.integers(0, c.H_q, 48),
                                                              r.integers(0, c.n_new, 48))}
                  | {(0, 0, 0), (c.B - 1, c.H_q - 1, c.n_new - 1)})
    run_chunk(K, c, rows=rows)


def test_chunk_bad_blocks_and_lengths_raise_flags(K):
    c = case(2, 4, 2, 64, "bf16", 20, 40, 90, 16)
    inp = synth.chunk_inputs(c)
    q = to_dev(inp["q"], "bf16")
    kp, vp = to_dev(inp["k_pool"], "bf16"), to_dev(inp["v_pool"], "bf16")
    table = inp["block_table"].copy()
    table[0, 0] = 10 ** 6                      # outside the pool
    K.attn_prefill_paged(q, kp, vp, to_dev_i32(table), to_dev_i32(inp["lens"]))
    assert K.attn_device_error_flags() & 2
    big = np.array([10 ** 6, -5], np.int32)    # past the table's capacity / negative
    K.attn_prefill_paged(q, kp, vp, to_dev_i32(inp["block_table"]), to_dev_i32(big))
    assert K.attn_device_error_flags() & (1 | 4) == (1 | 4)
