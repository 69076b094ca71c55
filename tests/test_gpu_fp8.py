"""GPU parity of the 8-bit (OCP FP8 E4M3) paged KV cache: quantizing append (bit-exact) and decode."""
import numpy as np
import pytest

import oracle
import synth
from helpers import extreme_queries, poison_table_tail, assert_lse_close, assert_stored_output, to_dev, to_dev_i32

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


SPECIAL = np.array([1.0625, 1.1875, -1.0625, 0.0, -0.0, 1e4, -1e4, 447.0, 449.0, 464.0, 1e-4, 0.0029296875,
                    0.015625, 0.0146484375, np.inf, -np.inf, np.nan, 0.3, -0.7, 3.0], dtype=np.float32)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("scales", [(1.0, 1.0), (0.37, 3.0)])
def test_fp8_append_image_is_bit_exact(K, dtype, scales):
    ks, vs = scales
    case = synth.DecodeCase("fp8", 5, 4, 2, 128, dtype, 0, 60, True, 100 + len(dtype), n_new=19)
    inp = synth.fp8_decode_inputs(case)
    kn, vn = inp["k_new"].copy(), inp["v_new"].copy()
    # special values (ties, saturation, subnormals, signed zero, inf, NaN) in the first rows
    flat_k = kn.reshape(-1)
    flat_v = vn.reshape(-1)
    sp = synth.to_storage(SPECIAL * np.float32(ks), dtype)
    flat_k[:len(sp)] = sp
    flat_v[-len(sp):] = synth.to_storage(SPECIAL * np.float32(vs), dtype)
    kp, vp = u8(inp["k_pool"]), u8(inp["v_pool"])
    table = to_dev_i32(inp["block_table"])
    K.kv_append_fp8(kp, vp, to_dev(kn, dtype), to_dev(vn, dtype), to_dev_i32(inp["lens"]), table, ks, vs)
    torch.cuda.synchronize()
    assert K.attn_device_error_flags() == 0
    cache = oracle.PagedCache(inp["k_pool"], inp["v_pool"], inp["block_table"])
    cache.append(oracle.quantize(kn, dtype, ks), oracle.quantize(vn, dtype, vs), inp["lens"])
    assert kp.cpu().numpy().tobytes() == cache.k.tobytes(), "K pool image differs"
    assert vp.cpu().numpy().tobytes() == cache.v.tobytes(), "V pool image differs"


def run_fp8(K, case, lens=None, ks=synth.FP8_K_SCALE, vs=synth.FP8_V_SCALE, heads=None, poison=False, edit=None):
    """Append + decode over pools of every finite E4M3 code (empty slots hold NaN
    codes), checked with the stored-output rule: the fp32-output call meets the
    bar, the 16-bit output is its round-to-nearest-even."""
    print(f"[fp8] {case} k_scale={ks} v_scale={vs}", flush=True)
    inp = synth.fp8_decode_inputs(case, lens=lens)
    if edit is not None:
        edit(inp, case.dtype)
    dt = case.dtype
    lens_d = to_dev_i32(inp["lens"])
    kp, vp = u8(inp["k_pool"]), u8(inp["v_pool"])
    table = to_dev_i32(inp["block_table"])
    q = to_dev(inp["q"], dt)
    K.kv_append_fp8(kp, vp, to_dev(inp["k_new"], dt), to_dev(inp["v_new"], dt), lens_d, table, ks, vs)
    seq = to_dev_i32(inp["lens"] + 1)
    if poison:  # the decode must read no table entry past a sequence's last block
        table = to_dev_i32(poison_table_tail(inp["block_table"], inp["lens"] + 1, kp.shape[0]))
    o, lse = K.attn_decode_paged_fp8(q, kp, vp, table, seq, k_scale=ks, v_scale=vs, scale=case.sm_scale,
                                     return_lse=True)
    o32 = K.attn_decode_paged_fp8(q, kp, vp, table, seq, k_scale=ks, v_scale=vs, scale=case.sm_scale,
                                  out_fp32=True)
    torch.cuda.synchronize()
    assert K.attn_device_error_flags() == 0
    cache = oracle.PagedCache(inp["k_pool"], inp["v_pool"], inp["block_table"])
    Oref, Lref = oracle.decode_step_fp8(cache, inp["q"], inp["k_new"], inp["v_new"], inp["lens"], case.sm_scale, dt,
                                        ks, vs, heads=heads)
    assert kp.cpu().numpy().tobytes() == cache.k.tobytes(), "K pool image differs"
    got_l = lse.cpu().numpy().astype(np.float64)
    if heads is not None:
        idx = tuple(np.array(heads).T)
        o, o32, Oref, got_l, Lref = o[idx], o32[idx], Oref[idx], got_l[idx], Lref[idx]
    mx, mean = assert_stored_output(o, o32, Oref, dt)
    assert_lse_close(got_l, Lref, dt)
    print(f"[fp8] fp32-output max-abs {mx:.3e} mean-abs {mean:.3e}", flush=True)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
def test_fp8_decode_chunk_boundaries(K, d, dtype):
    lens = np.array([0, 14, 15, 16, 30, 31, 255, 511, 512, 1023, 1500], dtype=np.int32)
    run_fp8(K, synth.DecodeCase("fp8", len(lens), 8, 2, d, dtype, 0, 1600, True, 110 + d), lens=lens)


@pytest.mark.parametrize("G", [1, 4, 8, 16, 24, 32])
def test_fp8_decode_gqa_groups(K, G):
    run_fp8(K, synth.DecodeCase("fp8", 3, 2 * G, 2, 128, "bf16", 1, 700, True, 120 + G))


def test_fp8_decode_workload(K):
    """The paged decode workload (B=64, H_q=32, H_kv=8, lengths 128 .. 8192) with an
    8-bit cache, every (sequence, head)."""
    run_fp8(K, synth.DECODE_PAGED)


def test_fp8_decode_other_scales(K):
    """Scales that are not powers of two (the append's fp32 reciprocal and the
    decode's scaling paths)."""
    run_fp8(K, synth.DecodeCase("fp8", 4, 8, 2, 128, "bf16", 1, 400, True, 140), ks=0.0123, vs=0.0031)


def test_fp8_bad_block_raises_flag(K):
    case = synth.DecodeCase("fp8", 2, 4, 2, 64, "bf16", 20, 40, True, 130)
    inp = synth.fp8_decode_inputs(case)
    table = inp["block_table"].copy()
    table[1, 0] = -7
    K.attn_decode_paged_fp8(to_dev(inp["q"], "bf16"), u8(inp["k_pool"]), u8(inp["v_pool"]), to_dev_i32(table),
                            to_dev_i32(inp["lens"] + 1))
    assert K.attn_device_error_flags() & 2


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_decode_reads_no_table_entry_past_the_length(K, d):
    lens = np.array([0, 1, 15, 16, 17, 31, 32, 33, 47, 48, 63, 64, 127, 128, 250], dtype=np.int32)
    run_fp8(K, synth.DecodeCase("f8", len(lens), 8, 2, d, "bf16", 0, 260, True, 300 + d), lens=lens, poison=True)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_fp8_decode_extreme_queries(K, dtype):
    """Query heads that are all zero, one dominant channel over tiny ones, tiny,
    or large, over the FP8 cache."""
    run_fp8(K, synth.DecodeCase("f8x", 4, 8, 2, 128, dtype, 1, 300, True, 340 + len(dtype)), edit=extreme_queries)
