"""attn_decode_paged_noalloc (the library's static workspace, no allocation) against
attn_decode_paged with a caller workspace, through the C ABI: two calls in a row, the
second smaller (the static array keeps the first call's contents), then a size
beyond the static workspace, which must be refused before anything is launched."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from helpers import assert_lse_close, assert_stored_output, bits_of, to_dev, to_dev_i32

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


def _one(K, case, lens=None):
    print(f"[noalloc] {case}", flush=True)
    inp = synth.decode_inputs(case, lens=lens)
    dt = case.dtype
    kp, vp = to_dev(inp["k_pool"], dt), to_dev(inp["v_pool"], dt)
    table = to_dev_i32(inp["block_table"])
    K.kv_append(kp, vp, to_dev(inp["k_new"], dt), to_dev(inp["v_new"], dt), to_dev_i32(inp["lens"]), table)
    q, seq = to_dev(inp["q"], dt), to_dev_i32(inp["lens"] + 1)
    o_ref, l_ref = K.attn_decode_paged(q, kp, vp, table, seq, scale=case.sm_scale, return_lse=True)
    o32_ref = K.attn_decode_paged(q, kp, vp, table, seq, scale=case.sm_scale, out_fp32=True)
    # the new entry point, called through the C ABI with preallocated outputs
    o = torch.empty_like(q)
    o32 = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    lse = torch.empty((case.B, case.H_q), dtype=torch.float32, device=q.device)
    L = K.lib()
    nb, H_kv, bs, d = kp.shape
    stream = torch.cuda.current_stream().cuda_stream
    for out, ls, f32 in ((o, lse, 0), (o32, None, 1)):
        rc = L.attn_decode_paged_noalloc(q.data_ptr(), kp.data_ptr(), vp.data_ptr(), table.data_ptr(), seq.data_ptr(),
                                         out.data_ptr(), ls.data_ptr() if ls is not None else None, case.B, case.H_q,
                                         H_kv, d, bs, table.shape[1], nb, case.sm_scale,
                                         K.DTYPE_CODES[q.dtype], f32, stream)
        assert rc == 0, L.attn_last_error().decode()
    torch.cuda.synchronize()
    assert K.attn_device_error_flags() == 0
    # the same kernels on the same inputs: the same bits as the call with a caller workspace
    assert np.array_equal(bits_of(o), bits_of(o_ref)), "16-bit output differs from attn_decode_paged"
    assert np.array_equal(bits_of(o32), bits_of(o32_ref)), "fp32 output differs from attn_decode_paged"
    assert np.array_equal(lse.cpu().numpy(), l_ref.cpu().numpy()), "lse differs from attn_decode_paged"
    # and the oracle's bar
    Oref, Lref = oracle.decode_step(oracle.PagedCache(inp["k_pool"], inp["v_pool"], inp["block_table"]), inp["q"],
                                    inp["k_new"], inp["v_new"], inp["lens"], case.sm_scale, dt)
    assert_stored_output(o, o32, Oref, dt)
    assert_lse_close(lse.cpu().numpy().astype(np.float64), Lref, dt)


def test_noalloc_matches_the_paged_decode_twice_second_call_smaller(K):
    _one(K, synth.DecodeCase("noalloc-1", 24, 32, 8, 128, "bf16", 100, 3000, True, 600))
    _one(K, synth.DecodeCase("noalloc-2", 3, 8, 2, 64, "f16", 0, 90, True, 601),
         lens=np.array([0, 17, 90], dtype=np.int32))


def test_noalloc_refuses_a_workspace_beyond_the_static_array(K):
    """The contiguous-decode workload's size as a paged table (B = 32, H_q = 64,
    32,784 tokens of capacity at d = 128) needs about 136 MB: refused, nothing launched."""
    L = K.lib()
    fake = 1 << 20  # 16-byte aligned; never dereferenced: the call fails validation first
    rc = L.attn_decode_paged_noalloc(fake, fake, fake, fake, fake, fake, None, 32, 64, 8, 128, 16, 2049, 40000,
                                     0.088, 2, 0, None)
    assert rc == 3, rc
    msg = L.attn_last_error().decode()
    assert "static scratch" in msg and "attn_decode_paged" in msg, msg
