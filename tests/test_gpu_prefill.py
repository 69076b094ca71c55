"""GPU parity of attn_prefill against the fp64 oracle (small and ragged shapes)."""
import numpy as np
import pytest

import oracle
import synth
from helpers import assert_close, assert_lse_close, bits_of, to_dev, values_of

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_flashattention_attn_amd as k
    k.lib()
    return k


def run_case(K, seed, B, H_q, H_kv, N, d, dtype, causal, out_fp32=False, scale=None, scale_by=1.0):
    print(f"[prefill] seed={seed} B={B} Hq={H_q} Hkv={H_kv} N={N} d={d} {dtype} causal={causal} "
          f"fp32out={out_fp32}", flush=True)
    raw = synth.random_prefill(seed, B, H_q, H_kv, N, d, dtype, scale_by=scale_by)
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    q, k, v = (to_dev(raw[n], dtype) for n in ("q", "k", "v"))
    o, lse = K.attn_prefill(q, k, v, causal=causal, scale=scale, return_lse=True, out_fp32=out_fp32)
    torch.cuda.synchronize()
    Q, Kk, V = (oracle.decode_bits(raw[n], dtype) for n in ("q", "k", "v"))
    Oref, Lref = oracle.one_shot(Q, Kk, V, scale, causal)
    assert_lse_close(lse.cpu().numpy().astype(np.float64), Lref, dtype)
    if dtype == "f32" or out_fp32:
        assert_close(values_of(o), Oref, dtype)
        return o
    # 16-bit output: the arithmetic (fp32-output mode) meets the bar on its own,
    # the stored output is exactly that result rounded to nearest-even, and so
    # differs from the oracle by at most the bar plus its own storage rounding.
    o32 = K.attn_prefill(q, k, v, causal=causal, scale=scale, out_fp32=True)
    torch.cuda.synchronize()
    assert_close(values_of(o32), Oref, dtype, what="O (fp32 output)")
    assert np.array_equal(bits_of(o), synth.to_storage(o32.cpu().numpy(), dtype)), \
        "16-bit output is not the round-to-nearest-even of the fp32 result"
    assert_close(values_of(o), Oref, dtype, storage_slack=True)
    return o


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 15, 17, 64, 129, 300])
def test_mfma_prefill_shapes(K, dtype, d, causal, N):
    run_case(K, 1000 + N + d, 1, 2, 2, N, d, dtype, causal)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("d", [16, 32, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_plain_prefill_shapes(K, dtype, d, causal):
    for N in (1, 17, 70):
        run_case(K, 2000 + N + d, 2, 2, 1, N, d, dtype, causal)


@pytest.mark.parametrize("G", [1, 4, 8])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_prefill(K, G, causal):
    run_case(K, 3000 + G, 2, 2 * G, 2, 200, 128, "bf16", causal)
    run_case(K, 3100 + G, 1, 2 * G, 2, 77, 16, "f32", causal)


@pytest.mark.parametrize("B,H_q,H_kv,N", [(1, 8, 8, 512), (1, 24, 8, 384), (3, 8, 2, 256), (1, 12, 4, 256),
                                          (2, 16, 4, 512), (1, 3, 1, 300)])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_block_orders(K, B, H_q, H_kv, N, causal):
    """Shapes that take every branch of the workgroup order (128-row query blocks,
    8 XCDs): blocks a multiple of 8 or not; causal with whole heads per XCD in
    groups of two (2, 16, 4, 512) or one (odd heads per XCD: 1 of 8 x 512,
    3 of 24 x 384, 3 of 3 x 8 x 256); causal with a per-XCD count that is not a
    multiple of the query blocks (1 x 12 x 256); the plain order (1 x 3 x 300).
    Every query block must be computed once, with its own head's K and V."""
    run_case(K, 5000 + B * H_q + N, B, H_q, H_kv, N, 128, "bf16", causal)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_gqa_small_noncausal_d64(K, dtype):
    """Small non-causal d = 64 problems take the key-split kernel: GQA head mapping
    and ragged tails through it."""
    run_case(K, 3200, 2, 8, 2, 200, 64, dtype, False)
    run_case(K, 3201, 1, 4, 1, 1000, 64, dtype, False)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("B,H_q,H_kv,N", [(1, 17, 17, 1900), (1, 16, 4, 2000), (2, 16, 4, 1100)])
def test_noncausal_d64_on_both_sides_of_the_kernel_switch(K, dtype, B, H_q, H_kv, N):
    """Non-causal d = 64 problems with fewer 128-row query blocks than the GPU has
    compute units (256) take the key-split kernel; the others take the main MFMA
    kernel.  Block counts here: 255 (key-split), 256 and 288 (main kernel), with
    GQA and ragged lengths."""
    run_case(K, 3300 + N + H_q, B, H_q, H_kv, N, 64, dtype, False)


def test_fp32_output_mode(K):
    """fp32 output separates arithmetic error from bf16 storage rounding."""
    o = run_case(K, 4000, 1, 4, 4, 513, 128, "bf16", True, out_fp32=True)
    assert o.dtype == torch.float32


def test_prefill_f32_exact_path_large_d(K):
    run_case(K, 4100, 1, 2, 2, 300, 128, "f32", True)
    run_case(K, 4101, 1, 2, 2, 300, 64, "f32", False)


def test_prefill_zero_and_negative_scale(K):
    run_case(K, 4200, 1, 2, 2, 40, 64, "bf16", True, scale=0.0)
    run_case(K, 4201, 1, 2, 2, 40, 64, "bf16", False, scale=-0.125)


def test_prefill_large_scores(K):
    """Scores in the hundreds: the running max keeps exp2 in range."""
    run_case(K, 4300, 1, 2, 2, 130, 64, "bf16", True, scale=1.0, scale_by=3.0)


def test_prefill_deterministic(K):
    raw = synth.random_prefill(5, 1, 4, 4, 700, 128, "bf16")
    q, k, v = (to_dev(raw[n], "bf16") for n in ("q", "k", "v"))
    o1 = K.attn_prefill(q, k, v, causal=True)
    o2 = K.attn_prefill(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
