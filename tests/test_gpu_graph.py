"""The compute calls under HIP graph capture: a serving loop may record a step
(append, then attention) once and replay it.  Each case runs the step eagerly,
records it into a graph, and replays the graph several times.  Before every
replay the outputs, lse and workspace are filled with NaN bytes by eager work
of the program, and after it they must hold exactly the eager step's bytes."""
import numpy as np
import pytest

import synth
from helpers import to_dev, to_dev_i32

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

REPLAYS = 4


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_flashattention_attn_amd as k
    k.lib()
    assert k.attn_device_error_flags() == 0
    return k


def poison(bufs):
    for b in bufs:
        b.view(torch.uint8).fill_(0xFF)


def replay_matches_eager(K, step, outs, scratch=(), kept=()):
    """step() writes `outs` (poisoned before each run), uses `scratch` (poisoned
    too) and appends into `kept` (caches: compared, never poisoned); eager bytes
    against every replay's."""
    poison(list(outs) + list(scratch))
    step()
    torch.cuda.synchronize()
    assert K.attn_device_error_flags() == 0
    outs = list(outs) + list(kept)
    ref = [o.view(torch.uint8).cpu().numpy().copy() for o in outs]
    # warm up on a side stream, then record (torch's capture recipe)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        poison(list(outs[:len(outs) - len(kept)]) + list(scratch))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert K.attn_device_error_flags() == 0
        for i, (o, rb) in enumerate(zip(outs, ref)):
            assert np.array_equal(o.view(torch.uint8).cpu().numpy(), rb), f"replay {r}: output {i} differs from eager"


def test_graph_paged_append_and_decode(K):
    c = synth.DecodeCase("graph", 8, 32, 8, 128, "bf16", 100, 2000, True, 610)
    print(f"[graph] paged append + decode {c}", flush=True)
    inp = synth.decode_inputs(c)
    q = to_dev(inp["q"], "bf16")
    kp, vp = to_dev(inp["k_pool"], "bf16"), to_dev(inp["v_pool"], "bf16")
    tb = to_dev_i32(inp["block_table"])
    lens, seq = to_dev_i32(inp["lens"]), to_dev_i32(inp["lens"] + 1)
    kn, vn = to_dev(inp["k_new"], "bf16"), to_dev(inp["v_new"], "bf16")
    ws = torch.empty(K.attn_decode_workspace_bytes(c.B, c.H_q, tb.shape[1] * 16, c.d), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((c.B, c.H_q), dtype=torch.float32, device="cuda")

    def step():
        K.kv_append(kp, vp, kn, vn, lens, tb)  # reads the lengths, never advances them: same rows each time
        K.attn_decode_paged(q, kp, vp, tb, seq, scale=c.sm_scale, return_lse=True, workspace=ws, out=o, lse=lse)

    replay_matches_eager(K, step, (o, lse), (ws,), (kp, vp))


def test_graph_contiguous_decode(K):
    c = synth.DecodeCase("graph", 4, 16, 4, 128, "f16", 0, 3000, False, 611)
    print(f"[graph] contiguous decode {c}", flush=True)
    inp = synth.decode_inputs(c)
    q = to_dev(inp["q"], "f16")
    kc, vc = to_dev(inp["k_cache"], "f16"), to_dev(inp["v_cache"], "f16")
    K.kv_append(kc, vc, to_dev(inp["k_new"], "f16"), to_dev(inp["v_new"], "f16"), to_dev_i32(inp["lens"]))
    seq = to_dev_i32(inp["lens"] + 1)
    ws = torch.empty(K.attn_decode_workspace_bytes(c.B, c.H_q, kc.shape[2], c.d), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((c.B, c.H_q), dtype=torch.float32, device="cuda")

    def step():
        K.attn_decode(q, kc, vc, seq, scale=c.sm_scale, return_lse=True, workspace=ws, out=o, lse=lse)

    replay_matches_eager(K, step, (o, lse), (ws,))


@pytest.mark.parametrize("fmt", ["fp8", "int8", "int4"])
def test_graph_quantised_decode(K, fmt):
    c = synth.DecodeCase("graph", 6, 16, 4, 128, "bf16", 0, 1500, True, 612 + len(fmt))
    print(f"[graph] {fmt} paged decode {c}", flush=True)
    gen = {"fp8": synth.fp8_decode_inputs, "int8": synth.int8_decode_inputs, "int4": synth.int4_decode_inputs}[fmt]
    inp = gen(c)
    q = to_dev(inp["q"], "bf16")
    dtype = np.int8 if fmt == "int8" else np.uint8
    kp = torch.from_numpy(np.ascontiguousarray(inp["k_pool"], dtype=dtype)).cuda()
    vp = torch.from_numpy(np.ascontiguousarray(inp["v_pool"], dtype=dtype)).cuda()
    tb = to_dev_i32(inp["block_table"])
    lens, seq = to_dev_i32(inp["lens"]), to_dev_i32(inp["lens"] + 1)
    kn, vn = to_dev(inp["k_new"], "bf16"), to_dev(inp["v_new"], "bf16")
    ws = torch.empty(K.attn_decode_workspace_bytes(c.B, c.H_q, tb.shape[1] * 16, c.d), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((c.B, c.H_q), dtype=torch.float32, device="cuda")
    if fmt == "fp8":
        def step():
            K.kv_append_fp8(kp, vp, kn, vn, lens, tb, synth.FP8_K_SCALE, synth.FP8_V_SCALE)
            K.attn_decode_paged_fp8(q, kp, vp, tb, seq, k_scale=synth.FP8_K_SCALE, v_scale=synth.FP8_V_SCALE,
                                    scale=c.sm_scale, return_lse=True, workspace=ws, out=o, lse=lse)
    else:
        ks = torch.from_numpy(inp["k_scales"]).cuda()
        vs = torch.from_numpy(inp["v_scales"]).cuda()
        app = K.kv_append_int8 if fmt == "int8" else K.kv_append_int4
        dec = K.attn_decode_paged_int8 if fmt == "int8" else K.attn_decode_paged_int4

        def step():
            app(kp, vp, kn, vn, lens, tb, ks, vs)
            dec(q, kp, vp, tb, seq, ks, vs, scale=c.sm_scale, return_lse=True, workspace=ws, out=o, lse=lse)

    replay_matches_eager(K, step, (o, lse), (ws,), (kp, vp))


@pytest.mark.parametrize("causal", [False, True])
def test_graph_prefill(K, causal):
    pc = synth.PrefillCase("graph", 2, 8, 2, 700, 128, "bf16", causal, True, 620 + causal)
    print(f"[graph] prefill {pc}", flush=True)
    inp = synth.prefill_inputs(pc)
    q, k, v = (to_dev(inp[n], "bf16") for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((pc.B, pc.H_q, pc.N), dtype=torch.float32, device="cuda")

    def step():
        K.attn_prefill(q, k, v, causal=causal, scale=pc.sm_scale, return_lse=True, out=o, lse=lse)

    replay_matches_eager(K, step, (o, lse))


def test_graph_chunk_prefill(K):
    c = synth.DecodeCase("graph", 4, 8, 2, 128, "bf16", 0, 900, True, 630, n_new=200)
    print(f"[graph] chunk prefill {c}", flush=True)
    inp = synth.chunk_inputs(c)
    lens = to_dev_i32(inp["lens"])
    q = to_dev(inp["q"], "bf16")
    kp, vp = to_dev(inp["k_pool"], "bf16"), to_dev(inp["v_pool"], "bf16")
    tb = to_dev_i32(inp["block_table"])
    kn, vn = to_dev(inp["k_new"], "bf16"), to_dev(inp["v_new"], "bf16")
    o = torch.empty_like(q)
    lse = torch.empty((c.B, c.H_q, c.n_new), dtype=torch.float32, device="cuda")

    def step():
        K.kv_append(kp, vp, kn, vn, lens, tb)
        K.attn_prefill_paged(q, kp, vp, tb, lens, scale=c.sm_scale, return_lse=True, out=o, lse=lse)

    replay_matches_eager(K, step, (o, lse), (), (kp, vp))
