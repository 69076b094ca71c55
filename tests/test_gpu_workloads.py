"""The five workloads at full size: GPU vs the fp64 oracle.

Every workload is compared element by element: every output row of the
prefills (O and lse) and every (sequence, head) of the decodes, and the whole
byte image of each cache after the append.
"""
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
    k.attn_device_error_flags()
    return k


def test_tiny_f32_prefill_then_16_decode_steps(K):
    c = synth.TINY_PREFILL
    print(f"[workload] {c.name}", flush=True)
    raw = synth.prefill_inputs(c)
    q, k, v = (to_dev(raw[n], c.dtype) for n in ("q", "k", "v"))
    o, lse = K.attn_prefill(q, k, v, causal=c.causal, scale=c.sm_scale, return_lse=True)
    Q, Kk, V = (oracle.decode_bits(raw[n], c.dtype) for n in ("q", "k", "v"))
    Oref, Lref = oracle.one_shot(Q, Kk, V, c.sm_scale, c.causal)
    torch.cuda.synchronize()
    assert_close(values_of(o), Oref, "f32")
    assert_lse_close(lse.cpu().numpy().astype(np.float64), Lref, "f32")

    # decode phase: seed the cache with the prefill K/V (one 64-token append), then 16 steps
    steps = synth.tiny_decode_steps(c)
    max_len = c.N + len(steps)
    kc = torch.zeros((c.B, c.H_kv, max_len, c.d), dtype=torch.float32, device="cuda")
    vc = torch.zeros_like(kc)
    K.kv_append(kc, vc, k, v, to_dev_i32(np.zeros(c.B, np.int32)))
    ocache = oracle.ContigCache(np.zeros((c.B, c.H_kv, max_len, c.d), np.float32),
                                np.zeros((c.B, c.H_kv, max_len, c.d), np.float32))
    ocache.append(raw["k"], raw["v"], np.zeros(c.B, np.int32))
    qs = []
    ks = [oracle.decode_bits(raw["k"][0, :, t], "f32") for t in range(c.N)]
    vs = [oracle.decode_bits(raw["v"][0, :, t], "f32") for t in range(c.N)]
    for t, st in enumerate(steps):
        L = c.N + t
        K.kv_append(kc, vc, to_dev(st["k_new"], "f32"), to_dev(st["v_new"], "f32"),
                    to_dev_i32(np.full(c.B, L, np.int32)))
        og, lg = K.attn_decode(to_dev(st["q"], "f32"), kc, vc, to_dev_i32(np.full(c.B, L + 1, np.int32)),
                               scale=c.sm_scale, return_lse=True)
        ocache.append(st["k_new"], st["v_new"], np.full(c.B, L, np.int32))
        ks.append(oracle.decode_bits(st["k_new"][0, :, 0], "f32"))
        vs.append(oracle.decode_bits(st["v_new"][0, :, 0], "f32"))
        qs.append(oracle.decode_bits(st["q"][0], "f32"))
        # the oracle's cached decoder over the whole token stream; its last step is this step
        Oc, _ = oracle.cached_decode([np.zeros_like(qs[0])] * L + [qs[-1]], ks, vs, c.sm_scale)
        torch.cuda.synchronize()
        assert_close(values_of(og)[0], Oc[-1], "f32", what=f"decode step {t}")
        Od, Ld = oracle.decode_step(oracle.ContigCache(bits_of(kc), bits_of(vc)), st["q"],
                                    np.zeros((1, c.H_kv, 0, c.d), np.float32),
                                    np.zeros((1, c.H_kv, 0, c.d), np.float32),
                                    np.full(c.B, L + 1, np.int32), c.sm_scale, "f32")
        assert_lse_close(lg.cpu().numpy().astype(np.float64), Ld, "f32")
    assert bits_of(kc).tobytes() == ocache.k.tobytes()
    assert bits_of(vc).tobytes() == ocache.v.tobytes()
    assert K.attn_device_error_flags() == 0


def test_f16_prefill_1x8x1024x64(K):
    c = synth.PREFILL_F16
    print(f"[workload] {c.name}", flush=True)
    raw = synth.prefill_inputs(c)
    q, k, v = (to_dev(raw[n], c.dtype) for n in ("q", "k", "v"))
    o, lse = K.attn_prefill(q, k, v, causal=c.causal, scale=c.sm_scale, return_lse=True)
    Q, Kk, V = (oracle.decode_bits(raw[n], c.dtype) for n in ("q", "k", "v"))
    Oref, Lref = oracle.one_shot(Q, Kk, V, c.sm_scale, c.causal)
    torch.cuda.synchronize()
    assert_close(values_of(o), Oref, c.dtype)
    assert_lse_close(lse.cpu().numpy().astype(np.float64), Lref, c.dtype)


def test_bf16_causal_prefill_4x32x4096x128(K):
    """Every output row (O and lse) of the causal workload against the fp64
    oracle, one (batch, head) at a time."""
    c = synth.PREFILL_BF16_CAUSAL
    print(f"[workload] {c.name}", flush=True)
    raw = synth.prefill_inputs(c)
    q, k, v = (to_dev(raw[n], c.dtype) for n in ("q", "k", "v"))
    o, lse = K.attn_prefill(q, k, v, causal=True, scale=c.sm_scale, return_lse=True)
    torch.cuda.synchronize()
    assert K.attn_device_error_flags() == 0
    og = bits_of(o)
    lg = lse.cpu().numpy().astype(np.float64)
    del o, lse, q, k, v
    mx, total, lmx = 0.0, 0.0, 0.0
    for b in range(c.B):
        for h in range(c.H_q):
            Q, Kk, V = (oracle.decode_bits(raw[n][b:b + 1, h:h + 1], c.dtype) for n in ("q", "k", "v"))
            Oref, Lref = oracle.one_shot(Q, Kk, V, c.sm_scale, causal=True)
            err = np.abs(oracle.decode_bits(og[b:b + 1, h:h + 1], c.dtype) - Oref)
            assert np.all(np.isfinite(err)), f"non-finite output at (b, h) = ({b}, {h})"
            assert float(err.max()) <= 1e-2, f"(b, h) = ({b}, {h}): max-abs {float(err.max()):.3e}"
            mx, total = max(mx, float(err.max())), total + float(err.sum())
            lmx = max(lmx, float(np.abs(lg[b:b + 1, h:h + 1] - Lref).max()))
    mean = total / og.size
    print(f"[workload] {c.name}: all {og.size // c.d} rows, O max-abs {mx:.3e} mean-abs {mean:.3e}, "
          f"lse max-abs {lmx:.3e}", flush=True)
    assert mean <= 1e-3, f"O mean-abs {mean:.3e}"
    assert lmx <= 1e-3, f"lse max-abs {lmx:.3e}"


def _decode_workload(K, c):
    print(f"[workload] {c.name}", flush=True)
    inp = synth.decode_inputs(c)
    dt = c.dtype
    lens = inp["lens"]
    q, kn, vn = to_dev(inp["q"], dt), to_dev(inp["k_new"], dt), to_dev(inp["v_new"], dt)
    if c.paged:
        kc, vc = to_dev(inp["k_pool"], dt), to_dev(inp["v_pool"], dt)
        table = to_dev_i32(inp["block_table"])
        K.kv_append(kc, vc, kn, vn, to_dev_i32(lens), table)
        o, lse = K.attn_decode_paged(q, kc, vc, table, to_dev_i32(lens + 1), scale=c.sm_scale, return_lse=True)
        ocache = oracle.PagedCache(inp["k_pool"], inp["v_pool"], inp["block_table"])
    else:
        kc, vc = to_dev(inp["k_cache"], dt), to_dev(inp["v_cache"], dt)
        K.kv_append(kc, vc, kn, vn, to_dev_i32(lens))
        o, lse = K.attn_decode(q, kc, vc, to_dev_i32(lens + 1), scale=c.sm_scale, return_lse=True)
        ocache = oracle.ContigCache(inp["k_cache"], inp["v_cache"])
    torch.cuda.synchronize()
    assert K.attn_device_error_flags() == 0
    # every (sequence, head) against the oracle
    Oref, Lref = oracle.decode_step(ocache, inp["q"], inp["k_new"], inp["v_new"], lens, c.sm_scale, dt)
    mx, mean = assert_close(values_of(o), Oref, dt)
    lg = lse.cpu().numpy().astype(np.float64)
    assert_lse_close(lg, Lref, dt)
    print(f"[workload] {c.name}: all {c.B * c.H_q} heads, O max-abs {mx:.3e} mean-abs {mean:.3e}, "
          f"lse max-abs {float(np.abs(lg - Lref).max()):.3e}", flush=True)
    # whole-buffer append images
    assert np.array_equal(bits_of(kc), ocache.k), "K cache image differs"
    assert np.array_equal(bits_of(vc), ocache.v), "V cache image differs"


def test_bf16_gqa_decode_contiguous_b32(K):
    _decode_workload(K, synth.DECODE_CONTIG)


def test_bf16_gqa_decode_paged_b64(K):
    _decode_workload(K, synth.DECODE_PAGED)
