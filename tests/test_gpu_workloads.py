"""The five workloads at full size: GPU vs the fp64 oracle.

Small workloads are compared element by element; the large ones on sampled
rows / heads that the oracle computes one by one, plus properties that hold at
any size (finite outputs; every output row is a convex combination of value
rows, so it lies inside their per-component range).
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


def _convex_hull_check(O, V, G):
    """Every O row of head h lies inside [min, max] of its KV head's value rows, per component."""
    vmin = V.amin(dim=2).repeat_interleave(G, dim=1)  # [B, H_q, d]
    vmax = V.amax(dim=2).repeat_interleave(G, dim=1)
    Of = O.float()
    tol = 1e-2
    assert bool(torch.all(Of >= vmin.float().unsqueeze(2) - tol))
    assert bool(torch.all(Of <= vmax.float().unsqueeze(2) + tol))


def test_bf16_causal_prefill_4x32x4096x128(K):
    c = synth.PREFILL_BF16_CAUSAL
    print(f"[workload] {c.name}", flush=True)
    raw = synth.prefill_inputs(c)
    q, k, v = (to_dev(raw[n], c.dtype) for n in ("q", "k", "v"))
    o, lse = K.attn_prefill(q, k, v, causal=True, scale=c.sm_scale, return_lse=True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    _convex_hull_check(o, v, 1)
    r = np.random.Generator(np.random.SFC64(123))
    rows = []
    for b in range(c.B):
        for h in r.choice(c.H_q, 4, replace=False):
            for i in [0, 1, 63, 64, 127, 128, 129, 2047, 2048, c.N - 1] + list(r.integers(0, c.N, 6)):
                rows.append((b, int(h), int(i)))
    Oref, Lref = oracle.attention_rows(_Lazy(raw["q"], c.dtype), _Lazy(raw["k"], c.dtype),
                                       _Lazy(raw["v"], c.dtype), c.sm_scale, rows, causal=True)
    og = values_of(o)
    lg = lse.cpu().numpy().astype(np.float64)
    got = np.stack([og[b, h, i] for b, h, i in rows])
    gotl = np.array([lg[b, h, i] for b, h, i in rows])
    assert_close(got, Oref, c.dtype)
    assert_lse_close(gotl, Lref, c.dtype)


class _Lazy:
    """Decodes storage bits to fp64 on slicing (so the oracle never holds the whole tensor)."""

    def __init__(self, bits, dtype):
        self.bits, self.dtype, self.shape = bits, dtype, bits.shape

    def __getitem__(self, idx):
        return oracle.decode_bits(self.bits[idx], self.dtype)


def _decode_workload(K, c, n_heads=24):
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
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    r = np.random.Generator(np.random.SFC64(321))
    bs = {int(np.argmin(lens)), int(np.argmax(lens))} | set(int(x) for x in r.choice(c.B, 6, replace=False))
    heads = sorted({(b, int(h)) for b in bs for h in r.choice(c.H_q, max(1, n_heads // len(bs)), replace=False)})
    Oref, Lref = oracle.decode_step(ocache, inp["q"], inp["k_new"], inp["v_new"], lens, c.sm_scale, dt,
                                    heads=heads)
    idx = tuple(np.array(heads).T)
    assert_close(values_of(o)[idx], Oref[idx], dt)
    assert_lse_close(lse.cpu().numpy().astype(np.float64)[idx], Lref[idx], dt)
    # whole-buffer append images
    assert np.array_equal(bits_of(kc), ocache.k), "K cache image differs"
    assert np.array_equal(bits_of(vc), ocache.v), "V cache image differs"


def test_bf16_gqa_decode_contiguous_b32(K):
    _decode_workload(K, synth.DECODE_CONTIG)


def test_bf16_gqa_decode_paged_b64(K):
    _decode_workload(K, synth.DECODE_PAGED)
