"""GPU parity of attn_prefill_fp8 (FP8 E4M3 Q, K, V with per-tensor scales) with the oracle."""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_close, assert_lse_close, values_of

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


def u8(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


TORCH_OUT = {"bf16": torch.bfloat16, "f16": torch.float16}


def run_fp8_prefill(K, case, causal, scales=(0.5, 0.25, 1.0), rows=None):
    print(f"[prefill fp8] {case} causal={causal} scales={scales}", flush=True)
    inp = synth.fp8_prefill_inputs(case)
    qs, ks, vs = scales
    scale = 1.0 / np.sqrt(case.d)
    o, lse = K.attn_prefill_fp8(u8(inp["q"]), u8(inp["k"]), u8(inp["v"]), causal=causal, scale=scale,
                                q_scale=qs, k_scale=ks, v_scale=vs, out_dtype=TORCH_OUT[case.dtype], return_lse=True)
    torch.cuda.synchronize()
    assert K.attn_device_error_flags() == 0
    Oref, Lref = oracle.prefill_fp8(inp["q"], inp["k"], inp["v"], qs, ks, vs, scale, causal, rows=rows)
    got_o, got_l = values_of(o), lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        idx = tuple(np.array(rows).T)
        got_o, got_l = got_o[idx], got_l[idx]
    assert_close(got_o, Oref, case.dtype)
    assert_lse_close(got_l, Lref, case.dtype)


def case(B, H_q, H_kv, N, d, dtype, seed):
    return synth.PrefillCase("fp8p", B, H_q, H_kv, N, d, dtype, True, True, seed)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_fp8_prefill_tiles_and_ragged_tail(K, d, dtype, causal):
    """Several 128-row query blocks and 64-key tiles, with a ragged tail (N = 300)."""
    run_fp8_prefill(K, case(2, 4, 2, 300, d, dtype, 300 + d), causal)


@pytest.mark.parametrize("N", [1, 63, 64, 65, 129, 517])
def test_fp8_prefill_lengths(K, N):
    run_fp8_prefill(K, case(1, 2, 1, N, 128, "bf16", 310 + N), True)


@pytest.mark.parametrize("G", [1, 4, 8])
def test_fp8_prefill_gqa(K, G):
    run_fp8_prefill(K, case(1, 2 * G, 2, 200, 128, "bf16", 320 + G), True, scales=(1.0, 1.0, 0.5))


def test_fp8_prefill_workload_sampled_rows(K):
    """The causal prefill workload (B=4, H=32, N=4096, d=128) with FP8 inputs, on sampled rows."""
    c = synth.PREFILL_BF16_CAUSAL
    r = np.random.Generator(np.random.SFC64(331))
    rows = sorted({(int(b), int(h), int(i)) for b, h, i in
                   zip(r.integers(0, c.B, 48), r.integers(0, c.H_q, 48), r.integers(0, c.N, 48))})
    rows += [(0, 0, 0), (c.B - 1, c.H_q - 1, c.N - 1)]
    run_fp8_prefill(K, c, True, rows=rows)
