"""Calls on different streams run side by side on the GPU: a paged decode over a
bf16 cache, one over an int8 cache and a causal prefill, each with its own
outputs and workspace, enqueued on three streams with no synchronisation
between them, three rounds in a row.  Every result must be the bytes the same
call gives alone on the default stream: the kernels keep no state between
calls beyond their arguments (the device error flags are set only on errors)."""
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


def poisoned(t):
    t.view(torch.uint8).fill_(0xFF)
    return t


def test_three_streams_match_one_stream(K):
    # paged decode, bf16 cache
    c = synth.DecodeCase("streams", 16, 32, 8, 128, "bf16", 100, 3000, True, 640)
    print(f"[streams] {c}", flush=True)
    inp = synth.decode_inputs(c)
    q1 = to_dev(inp["q"], "bf16")
    kp, vp = to_dev(inp["k_pool"], "bf16"), to_dev(inp["v_pool"], "bf16")
    tb1 = to_dev_i32(inp["block_table"])
    K.kv_append(kp, vp, to_dev(inp["k_new"], "bf16"), to_dev(inp["v_new"], "bf16"), to_dev_i32(inp["lens"]), tb1)
    seq1 = to_dev_i32(inp["lens"] + 1)
    ws1 = torch.empty(K.attn_decode_workspace_bytes(c.B, c.H_q, tb1.shape[1] * 16, c.d), dtype=torch.uint8,
                      device="cuda")
    # paged decode, int8 cache
    c8 = synth.DecodeCase("streams", 12, 32, 8, 128, "bf16", 0, 2500, True, 641)
    print(f"[streams] int8 {c8}", flush=True)
    i8 = synth.int8_decode_inputs(c8)
    q2 = to_dev(i8["q"], "bf16")
    k8 = torch.from_numpy(np.ascontiguousarray(i8["k_pool"], dtype=np.int8)).cuda()
    v8 = torch.from_numpy(np.ascontiguousarray(i8["v_pool"], dtype=np.int8)).cuda()
    ks, vs = torch.from_numpy(i8["k_scales"]).cuda(), torch.from_numpy(i8["v_scales"]).cuda()
    tb2 = to_dev_i32(i8["block_table"])
    K.kv_append_int8(k8, v8, to_dev(i8["k_new"], "bf16"), to_dev(i8["v_new"], "bf16"), to_dev_i32(i8["lens"]), tb2,
                     ks, vs)
    seq2 = to_dev_i32(i8["lens"] + 1)
    ws2 = torch.empty(K.attn_decode_workspace_bytes(c8.B, c8.H_q, tb2.shape[1] * 16, c8.d), dtype=torch.uint8,
                      device="cuda")
    # causal prefill
    pc = synth.PrefillCase("streams", 2, 16, 4, 1500, 128, "bf16", True, True, 642)
    print(f"[streams] prefill {pc}", flush=True)
    pinp = synth.prefill_inputs(pc)
    q3, k3, v3 = (to_dev(pinp[n], "bf16") for n in ("q", "k", "v"))

    def calls(outs):
        (o1, l1), (o2, l2), (o3, l3) = outs
        return [
            lambda: K.attn_decode_paged(q1, kp, vp, tb1, seq1, scale=c.sm_scale, return_lse=True, workspace=ws1,
                                        out=o1, lse=l1),
            lambda: K.attn_decode_paged_int8(q2, k8, v8, tb2, seq2, ks, vs, scale=c8.sm_scale, return_lse=True,
                                             workspace=ws2, out=o2, lse=l2),
            lambda: K.attn_prefill(q3, k3, v3, causal=True, scale=pc.sm_scale, return_lse=True, out=o3, lse=l3),
        ]

    def fresh():
        return [(poisoned(torch.empty_like(q1)), poisoned(torch.empty((c.B, c.H_q), device="cuda"))),
                (poisoned(torch.empty_like(q2)), poisoned(torch.empty((c8.B, c8.H_q), device="cuda"))),
                (poisoned(torch.empty_like(q3)), poisoned(torch.empty((pc.B, pc.H_q, pc.N), device="cuda")))]

    # one at a time on the default stream
    ref_outs = fresh()
    for f in calls(ref_outs):
        f()
        torch.cuda.synchronize()
    assert K.attn_device_error_flags() == 0
    ref = [[t.view(torch.uint8).cpu().numpy() for t in pair] for pair in ref_outs]

    streams = [torch.cuda.Stream() for _ in range(3)]
    for r in range(3):
        outs = fresh()
        poisoned(ws1), poisoned(ws2)
        torch.cuda.synchronize()
        for s, f in zip(streams, calls(outs)):
            with torch.cuda.stream(s):
                f()
        torch.cuda.synchronize()
        assert K.attn_device_error_flags() == 0
        for i, (pair, rp) in enumerate(zip(outs, ref)):
            for t, rb in zip(pair, rp):
                assert np.array_equal(t.view(torch.uint8).cpu().numpy(), rb), f"round {r}: call {i} differs"
