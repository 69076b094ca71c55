"""Every output element is written and no stale workspace content leaks in:
each call gets its output, lse and workspace filled with NaN bytes (0xFF) and
must return exactly what the same call returns into fresh buffers."""
import numpy as np
import pytest

import synth
from helpers import to_dev, to_dev_i32

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


def nan_like(t):
    p = torch.empty_like(t)
    p.view(torch.uint8).fill_(0xFF)
    return p


def same(a, b, what):
    assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{what}: differs with poisoned buffers"


def check_decode(K, fn, q, ws_bytes, lse_shape, **kw):
    """fn(out=, lse=, workspace=, return_lse=True) -> (o, lse); compare fresh and poisoned buffers."""
    o0, l0 = fn(return_lse=True, **kw)
    out = nan_like(o0)
    lse = torch.empty(lse_shape, dtype=torch.float32, device=q.device)
    lse.view(torch.uint8).fill_(0xFF)
    ws = torch.full((ws_bytes,), 0xFF, dtype=torch.uint8, device=q.device)
    o1, l1 = fn(return_lse=True, out=out, lse=lse, workspace=ws, **kw)
    torch.cuda.synchronize()
    assert K.attn_device_error_flags() == 0
    same(o0, o1, "O")
    same(l0, l1, "lse")
    assert torch.isfinite(o1.float()).all(), "O has non-finite values"


@pytest.mark.parametrize("causal", [False, True])
def test_prefill_poisoned_outputs(K, causal):
    pc = synth.PrefillCase("poison", 2, 8, 2, 300, 128, "bf16", causal, True, 400 + causal)
    inp = synth.prefill_inputs(pc)
    q, k, v = (to_dev(inp[n], "bf16") for n in ("q", "k", "v"))
    o0, l0 = K.attn_prefill(q, k, v, causal=causal, scale=pc.sm_scale, return_lse=True)
    o1, l1 = K.attn_prefill(q, k, v, causal=causal, scale=pc.sm_scale, return_lse=True, out=nan_like(o0),
                            lse=nan_like(l0))
    torch.cuda.synchronize()
    same(o0, o1, "O")
    same(l0, l1, "lse")


@pytest.mark.parametrize("paged", [False, True])
def test_decode_poisoned_buffers(K, paged):
    c = synth.DecodeCase("poison", 6, 16, 4, 128, "bf16", 0, 900, paged, 410 + paged)
    inp = synth.decode_inputs(c)
    q = to_dev(inp["q"], "bf16")
    seq = to_dev_i32(inp["lens"] + 1)
    if paged:
        kp, vp = to_dev(inp["k_pool"], "bf16"), to_dev(inp["v_pool"], "bf16")
        tb = to_dev_i32(inp["block_table"])
        K.kv_append(kp, vp, to_dev(inp["k_new"], "bf16"), to_dev(inp["v_new"], "bf16"), to_dev_i32(inp["lens"]), tb)
        ws = K.attn_decode_workspace_bytes(c.B, c.H_q, tb.shape[1] * 16, c.d)
        check_decode(K, lambda **kw: K.attn_decode_paged(q, kp, vp, tb, seq, scale=c.sm_scale, **kw), q, ws,
                     (c.B, c.H_q))
    else:
        kc, vc = to_dev(inp["k_cache"], "bf16"), to_dev(inp["v_cache"], "bf16")
        K.kv_append(kc, vc, to_dev(inp["k_new"], "bf16"), to_dev(inp["v_new"], "bf16"), to_dev_i32(inp["lens"]))
        ws = K.attn_decode_workspace_bytes(c.B, c.H_q, kc.shape[2], c.d)
        check_decode(K, lambda **kw: K.attn_decode(q, kc, vc, seq, scale=c.sm_scale, **kw), q, ws, (c.B, c.H_q))


@pytest.mark.parametrize("fmt", ["fp8", "int8", "int4"])
def test_quantised_decode_poisoned_buffers(K, fmt):
    c = synth.DecodeCase("poison", 6, 16, 4, 128, "bf16", 0, 900, True, 420 + len(fmt))
    gen = {"fp8": synth.fp8_decode_inputs, "int8": synth.int8_decode_inputs, "int4": synth.int4_decode_inputs}[fmt]
    inp = gen(c)
    q = to_dev(inp["q"], "bf16")
    dtype = np.int8 if fmt == "int8" else np.uint8
    kp = torch.from_numpy(np.ascontiguousarray(inp["k_pool"], dtype=dtype)).cuda()
    vp = torch.from_numpy(np.ascontiguousarray(inp["v_pool"], dtype=dtype)).cuda()
    tb = to_dev_i32(inp["block_table"])
    lens = to_dev_i32(inp["lens"])
    kn, vn = to_dev(inp["k_new"], "bf16"), to_dev(inp["v_new"], "bf16")
    seq = to_dev_i32(inp["lens"] + 1)
    ws = K.attn_decode_workspace_bytes(c.B, c.H_q, tb.shape[1] * 16, c.d)
    if fmt == "fp8":
        K.kv_append_fp8(kp, vp, kn, vn, lens, tb, synth.FP8_K_SCALE, synth.FP8_V_SCALE)
        fn = lambda **kw: K.attn_decode_paged_fp8(q, kp, vp, tb, seq, k_scale=synth.FP8_K_SCALE,  # noqa: E731
                                                  v_scale=synth.FP8_V_SCALE, scale=c.sm_scale, **kw)
    else:
        ks = torch.from_numpy(inp["k_scales"]).cuda()
        vs = torch.from_numpy(inp["v_scales"]).cuda()
        app = K.kv_append_int8 if fmt == "int8" else K.kv_append_int4
        dec = K.attn_decode_paged_int8 if fmt == "int8" else K.attn_decode_paged_int4
        app(kp, vp, kn, vn, lens, tb, ks, vs)
        fn = lambda **kw: dec(q, kp, vp, tb, seq, ks, vs, scale=c.sm_scale, **kw)  # noqa: E731
    check_decode(K, fn, q, ws, (c.B, c.H_q))


def test_chunk_prefill_poisoned_outputs(K):
    c = synth.DecodeCase("poison", 4, 8, 2, 128, "bf16", 0, 400, True, 430, n_new=70)
    inp = synth.chunk_inputs(c)
    lens = to_dev_i32(inp["lens"])
    q = to_dev(inp["q"], "bf16")
    kp, vp = to_dev(inp["k_pool"], "bf16"), to_dev(inp["v_pool"], "bf16")
    tb = to_dev_i32(inp["block_table"])
    K.kv_append(kp, vp, to_dev(inp["k_new"], "bf16"), to_dev(inp["v_new"], "bf16"), lens, tb)
    o0, l0 = K.attn_prefill_paged(q, kp, vp, tb, lens, scale=c.sm_scale, return_lse=True)
    o1, l1 = K.attn_prefill_paged(q, kp, vp, tb, lens, scale=c.sm_scale, return_lse=True, out=nan_like(o0),
                                  lse=nan_like(l0))
    torch.cuda.synchronize()
    assert K.attn_device_error_flags() == 0
    same(o0, o1, "O")
    same(l0, l1, "lse")


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_prefill_poisoned_outputs(K, causal):
    pc = synth.PrefillCase("poison", 1, 4, 2, 300, 128, "bf16", causal, True, 440 + causal)
    inp = synth.fp8_prefill_inputs(pc)
    q8, k8, v8 = (torch.from_numpy(np.ascontiguousarray(inp[n], dtype=np.uint8)).cuda() for n in ("q", "k", "v"))
    kw = dict(causal=causal, scale=pc.sm_scale, q_scale=synth.FP8_Q_SCALE, k_scale=synth.FP8_K_SCALE,
              v_scale=synth.FP8_V_SCALE)
    o0, l0 = K.attn_prefill_fp8(q8, k8, v8, return_lse=True, **kw)
    o1, l1 = K.attn_prefill_fp8(q8, k8, v8, return_lse=True, out=nan_like(o0), lse=nan_like(l0), **kw)
    torch.cuda.synchronize()
    assert K.attn_device_error_flags() == 0
    same(o0, o1, "O")
    same(l0, l1, "lse")
