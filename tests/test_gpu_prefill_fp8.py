"""GPU parity of attn_prefill_fp8 (FP8 E4M3 Q, K, V with per-tensor scales) with the oracle."""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_stored_output

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


def fp8_mfma_logit_shift(qv: np.ndarray, kv: np.ndarray) -> np.ndarray:
    """|exact dot product - what gfx950's FP8 matrix core returns| for raw E4M3
    values qv [Nq, d] and kv [Nk, d], per (query, key).

    Measured property of v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3): the
    products of each group of 8 consecutive bytes of a lane's operand (here 8
    consecutive d) are each cut toward zero to a multiple of 2^(E - 13), where
    2^E <= the group's largest |product| < 2^(E + 1), and then summed; products
    are otherwise exact.  With codes across the whole E4M3 range a logit can
    therefore move by a few 1e-3, which the lse shows directly."""
    nq, d = qv.shape
    p = (qv[:, None, :] * kv[None, :, :]).reshape(nq, kv.shape[0], d // 8, 8)
    mx = np.abs(p).max(axis=3, keepdims=True)
    gran = np.exp2(np.floor(np.log2(np.where(mx > 0, mx, 1.0))) - 13)
    cut = np.trunc(p / gran) * gran
    return np.abs((p - cut).sum(axis=(2, 3)))


def lse_tolerance(inp, qs, ks, scale, causal, rows):
    """Per output row: the lse bar plus the largest logit shift of fp8_mfma_logit_shift
    over the row's visible keys (lse moves by at most the largest logit move)."""
    qv, kv = oracle.e4m3_value(inp["q"]), oracle.e4m3_value(inp["k"])
    H_q, H_kv, N = qv.shape[1], kv.shape[1], qv.shape[2]
    tol = np.zeros(len(rows))
    by_head = {}
    for r, (b, h, i) in enumerate(rows):
        by_head.setdefault((b, h), []).append((r, i))
    for (b, h), items in by_head.items():
        g = h // (H_q // H_kv)
        idx = np.array([i for _, i in items])
        shift = fp8_mfma_logit_shift(qv[b, h, idx], kv[b, g]) * (scale * qs * ks)
        if causal:
            shift = np.where(np.arange(N)[None, :] <= idx[:, None], shift, 0.0)
        tol[[r for r, _ in items]] = 1e-3 + shift.max(axis=1)
    return tol


def run_fp8_prefill(K, case, causal, scales=(synth.FP8_Q_SCALE, synth.FP8_K_SCALE, synth.FP8_V_SCALE), rows=None):
    """FP8 prefill over Q, K, V spanning every finite E4M3 code, checked with the
    stored-output rule (fp32-output call within the bar; 16-bit output its
    round-to-nearest-even)."""
    print(f"[prefill fp8] {case} causal={causal} scales={scales}", flush=True)
    inp = synth.fp8_prefill_inputs(case)
    qs, ks, vs = scales
    scale = 1.0 / np.sqrt(case.d)
    q8, k8, v8 = u8(inp["q"]), u8(inp["k"]), u8(inp["v"])
    kw = dict(causal=causal, scale=scale, q_scale=qs, k_scale=ks, v_scale=vs, out_dtype=TORCH_OUT[case.dtype])
    o, lse = K.attn_prefill_fp8(q8, k8, v8, return_lse=True, **kw)
    o32 = K.attn_prefill_fp8(q8, k8, v8, out_fp32=True, **kw)
    torch.cuda.synchronize()
    assert K.attn_device_error_flags() == 0
    Oref, Lref = oracle.prefill_fp8(inp["q"], inp["k"], inp["v"], qs, ks, vs, scale, causal, rows=rows)
    got_l = lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        idx = tuple(np.array(rows).T)
        o, o32, got_l = o[idx], o32[idx], got_l[idx]
    else:
        rows = [(b, h, i) for b in range(case.B) for h in range(case.H_q) for i in range(case.N)]
        got_l, Lref = got_l.reshape(-1), Lref.reshape(-1)
    mx, mean = assert_stored_output(o, o32, Oref, case.dtype)
    # lse: the bar plus the matrix core's own rounding of the logits, row by row
    tol = lse_tolerance(inp, qs, ks, scale, causal, rows)
    lerr = np.abs(got_l - Lref)
    assert np.all(np.isfinite(got_l)), "lse: non-finite values"
    assert np.all(lerr <= tol), f"lse: max excess {float((lerr - tol).max()):.3e} over the per-row bound"
    print(f"[prefill fp8] fp32-output max-abs {mx:.3e} mean-abs {mean:.3e}; lse max-abs {lerr.max():.3e} "
          f"(rows whose bound exceeds 1e-3: {int(np.sum(tol > 1e-3 + 1e-12))} of {len(tol)}, "
          f"largest bound {tol.max():.3e})", flush=True)


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
    run_fp8_prefill(K, case(1, 2 * G, 2, 200, 128, "bf16", 320 + G), True)


def test_fp8_prefill_other_scales(K):
    run_fp8_prefill(K, case(1, 4, 2, 300, 128, "bf16", 340), True, scales=(0.011, 0.023, 0.0029))


def test_fp8_prefill_workload_sampled_rows(K):
    """The causal prefill workload (B=4, H=32, N=4096, d=128) with FP8 inputs, on sampled rows."""
    c = synth.PREFILL_BF16_CAUSAL
    r = np.random.Generator(np.random.SFC64(331))
    rows = sorted({(int(b), int(h), int(i)) for b, h, i in
                   zip(r.integers(0, c.B, 48), r.integers(0, c.H_q, 48), r.integers(0, c.N, 48))})
    rows += [(0, 0, 0), (c.B - 1, c.H_q - 1, c.N - 1)]
    run_fp8_prefill(K, c, True, rows=rows)
