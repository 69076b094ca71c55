"""GPU parity of the int8 and int4 paged KV caches with per-channel scales:
quantizing append (bit-exact) and decode."""
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


def i8(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int8)).cuda()


def f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


# multiples of the scale: ties (k + 0.5), saturation, zero, tiny, inf, NaN
SPECIAL = np.array([2.5, 3.5, -2.5, -0.5, 0.5, 126.5, 127.5, 300.0, -300.0, 0.0, -0.0, 1e-30, np.inf, -np.inf,
                    np.nan, 0.3, -0.7, 64.0], dtype=np.float32)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("pow2", [True, False])
def test_int8_append_image_is_bit_exact(K, dtype, pow2):
    case = synth.DecodeCase("i8", 5, 4, 2, 128, dtype, 0, 60, True, 200 + len(dtype), n_new=19)
    inp = synth.int8_decode_inputs(case)
    ks, vs = inp["k_scales"].copy(), inp["v_scales"].copy()
    if pow2:  # power-of-two scales make the tie values exact in every input type
        ks, vs = np.exp2(np.round(np.log2(ks))).astype(np.float32), np.exp2(np.round(np.log2(vs))).astype(np.float32)
    kn, vn = inp["k_new"].copy(), inp["v_new"].copy()
    # special multiples of each channel's scale in the first tokens of sequence 0, head 0
    n = len(SPECIAL)
    kn[0, 0, 0, :n] = synth.to_storage(SPECIAL * ks[0, :n], dtype)
    vn[0, 0, 1, :n] = synth.to_storage(SPECIAL * vs[0, :n], dtype)
    kp, vp = i8(inp["k_pool"]), i8(inp["v_pool"])
    table = to_dev_i32(inp["block_table"])
    K.kv_append_int8(kp, vp, to_dev(kn, dtype), to_dev(vn, dtype), to_dev_i32(inp["lens"]), table, f32(ks), f32(vs))
    torch.cuda.synchronize()
    assert K.attn_device_error_flags() == 0
    cache = oracle.PagedCache(inp["k_pool"], inp["v_pool"], inp["block_table"])
    kq = np.stack([oracle.quantize_int8(kn[b], dtype, ks) for b in range(case.B)])
    vq = np.stack([oracle.quantize_int8(vn[b], dtype, vs) for b in range(case.B)])
    cache.append(kq, vq, inp["lens"])
    if pow2 and dtype != "f16":  # the specials landed as intended (f16 flushes some products)
        assert kq[0, 0, 0, :3].tolist() == [2, 4, -2]
    assert kp.cpu().numpy().tobytes() == cache.k.tobytes(), "K pool image differs"
    assert vp.cpu().numpy().tobytes() == cache.v.tobytes(), "V pool image differs"


def run_int8(K, case, lens=None, heads=None, poison=False, edit=None):
    print(f"[int8] {case}", flush=True)
    inp = synth.int8_decode_inputs(case, lens=lens)
    if edit is not None:
        edit(inp, case.dtype)
    dt = case.dtype
    lens_d = to_dev_i32(inp["lens"])
    kp, vp = i8(inp["k_pool"]), i8(inp["v_pool"])
    ks, vs = f32(inp["k_scales"]), f32(inp["v_scales"])
    table = to_dev_i32(inp["block_table"])
    q = to_dev(inp["q"], dt)
    K.kv_append_int8(kp, vp, to_dev(inp["k_new"], dt), to_dev(inp["v_new"], dt), lens_d, table, ks, vs)
    seq = to_dev_i32(inp["lens"] + 1)
    if poison:  # the decode must read no table entry past a sequence's last block
        table = to_dev_i32(poison_table_tail(inp["block_table"], inp["lens"] + 1, kp.shape[0]))
    o, lse = K.attn_decode_paged_int8(q, kp, vp, table, seq, ks, vs, scale=case.sm_scale, return_lse=True)
    o32 = K.attn_decode_paged_int8(q, kp, vp, table, seq, ks, vs, scale=case.sm_scale, out_fp32=True)
    torch.cuda.synchronize()
    assert K.attn_device_error_flags() == 0
    cache = oracle.PagedCache(inp["k_pool"], inp["v_pool"], inp["block_table"])
    Oref, Lref = oracle.decode_step_int8(cache, inp["q"], inp["k_new"], inp["v_new"], inp["lens"], case.sm_scale, dt,
                                         inp["k_scales"], inp["v_scales"], heads=heads)
    assert kp.cpu().numpy().tobytes() == cache.k.tobytes(), "K pool image differs"
    got_l = lse.cpu().numpy().astype(np.float64)
    if heads is not None:
        idx = tuple(np.array(heads).T)
        o, o32, Oref, got_l, Lref = o[idx], o32[idx], Oref[idx], got_l[idx], Lref[idx]
    assert_stored_output(o, o32, Oref, dt)
    assert_lse_close(got_l, Lref, dt)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
def test_int8_decode_chunk_boundaries(K, d, dtype):
    lens = np.array([0, 14, 15, 16, 30, 31, 255, 511, 512, 1023, 1500], dtype=np.int32)
    run_int8(K, synth.DecodeCase("i8", len(lens), 8, 2, d, dtype, 0, 1600, True, 210 + d), lens=lens)


@pytest.mark.parametrize("G", [1, 4, 8, 16, 24, 32])
def test_int8_decode_gqa_groups(K, G):
    run_int8(K, synth.DecodeCase("i8", 3, 2 * G, 2, 128, "bf16", 1, 700, True, 220 + G))


def test_int8_decode_workload(K):
    """The paged decode workload (B=64, H_q=32, H_kv=8, lengths 128 .. 8192) with an
    int8 cache, every (sequence, head)."""
    run_int8(K, synth.DECODE_PAGED)


def test_int8_bad_block_raises_flag(K):
    case = synth.DecodeCase("i8", 2, 4, 2, 64, "bf16", 20, 40, True, 230)
    inp = synth.int8_decode_inputs(case)
    table = inp["block_table"].copy()
    table[1, 0] = -7
    K.attn_decode_paged_int8(to_dev(inp["q"], "bf16"), i8(inp["k_pool"]), i8(inp["v_pool"]), to_dev_i32(table),
                             to_dev_i32(inp["lens"] + 1), f32(inp["k_scales"]), f32(inp["v_scales"]))
    assert K.attn_device_error_flags() & 2


# ---------------------------------------------------------------- int4
SPECIAL4 = np.array([2.5, 3.5, -2.5, -0.5, 0.5, 6.5, 7.5, 30.0, -30.0, 0.0, -0.0, 1e-30, np.inf, -np.inf,
                     np.nan, 0.3, -0.7, 4.0], dtype=np.float32)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("pow2", [True, False])
@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_int4_append_image_is_bit_exact(K, dtype, pow2, d):
    """Both pools byte for byte after a 19-token append, V in the pool's operand
    order (runs of d / 8 bytes) at every head dimension the append takes."""
    case = synth.DecodeCase("i4", 5, 4, 2, d, dtype, 0, 60, True, 240 + len(dtype) + d, n_new=19)
    inp = synth.int4_decode_inputs(case)
    ks, vs = inp["k_scales"].copy(), inp["v_scales"].copy()
    if pow2:
        ks, vs = np.exp2(np.round(np.log2(ks))).astype(np.float32), np.exp2(np.round(np.log2(vs))).astype(np.float32)
    kn, vn = inp["k_new"].copy(), inp["v_new"].copy()
    n = len(SPECIAL4)
    kn[0, 0, 0, :n] = synth.to_storage(SPECIAL4 * ks[0, :n], dtype)
    vn[0, 0, 1, 3:3 + n] = synth.to_storage(SPECIAL4 * vs[0, 3:3 + n], dtype)  # odd offset: high nibbles too
    kp, vp = u8(inp["k_pool"]), u8(inp["v_pool"])
    table = to_dev_i32(inp["block_table"])
    K.kv_append_int4(kp, vp, to_dev(kn, dtype), to_dev(vn, dtype), to_dev_i32(inp["lens"]), table, f32(ks), f32(vs))
    torch.cuda.synchronize()
    assert K.attn_device_error_flags() == 0
    # the oracle's cache in row order (V's pool order undone), the append, then V back
    cache = oracle.PagedCache(inp["k_pool"], oracle.int4_v_from_pool(inp["v_pool"]), inp["block_table"])
    kq = np.stack([oracle.pack_int4(oracle.quantize_int4(kn[b], dtype, ks)) for b in range(case.B)])
    vq = np.stack([oracle.pack_int4(oracle.quantize_int4(vn[b], dtype, vs)) for b in range(case.B)])
    cache.append(kq, vq, inp["lens"])
    if pow2:
        assert oracle.quantize_int4(kn[0], dtype, ks)[0, 0, :7].tolist() == [2, 4, -2, 0, 0, 6, 7]
    assert kp.cpu().numpy().tobytes() == cache.k.tobytes(), "K pool image differs"
    assert vp.cpu().numpy().tobytes() == oracle.int4_v_to_pool(cache.v).tobytes(), "V pool image differs"


def u8(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).cuda()


def run_int4(K, case, lens=None, heads=None, poison=False, edit=None):
    print(f"[int4] {case}", flush=True)
    inp = synth.int4_decode_inputs(case, lens=lens)
    if edit is not None:
        edit(inp, case.dtype)
    dt = case.dtype
    lens_d = to_dev_i32(inp["lens"])
    kp, vp = u8(inp["k_pool"]), u8(inp["v_pool"])
    ks, vs = f32(inp["k_scales"]), f32(inp["v_scales"])
    table = to_dev_i32(inp["block_table"])
    q = to_dev(inp["q"], dt)
    K.kv_append_int4(kp, vp, to_dev(inp["k_new"], dt), to_dev(inp["v_new"], dt), lens_d, table, ks, vs)
    seq = to_dev_i32(inp["lens"] + 1)
    if poison:  # the decode must read no table entry past a sequence's last block
        table = to_dev_i32(poison_table_tail(inp["block_table"], inp["lens"] + 1, kp.shape[0]))
    o, lse = K.attn_decode_paged_int4(q, kp, vp, table, seq, ks, vs, scale=case.sm_scale, return_lse=True)
    o32 = K.attn_decode_paged_int4(q, kp, vp, table, seq, ks, vs, scale=case.sm_scale, out_fp32=True)
    torch.cuda.synchronize()
    assert K.attn_device_error_flags() == 0
    cache = oracle.PagedCache(inp["k_pool"], inp["v_pool"], inp["block_table"])
    Oref, Lref = oracle.decode_step_int4(cache, inp["q"], inp["k_new"], inp["v_new"], inp["lens"], case.sm_scale, dt,
                                         inp["k_scales"], inp["v_scales"], heads=heads)
    assert kp.cpu().numpy().tobytes() == cache.k.tobytes(), "K pool image differs"
    assert vp.cpu().numpy().tobytes() == cache.v.tobytes(), "V pool image differs"
    got_l = lse.cpu().numpy().astype(np.float64)
    if heads is not None:
        idx = tuple(np.array(heads).T)
        o, o32, Oref, got_l, Lref = o[idx], o32[idx], Oref[idx], got_l[idx], Lref[idx]
    assert_stored_output(o, o32, Oref, dt)
    assert_lse_close(got_l, Lref, dt)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
def test_int4_decode_chunk_boundaries(K, d, dtype):
    lens = np.array([0, 14, 15, 16, 30, 31, 255, 511, 512, 1023, 1500], dtype=np.int32)
    run_int4(K, synth.DecodeCase("i4", len(lens), 8, 2, d, dtype, 0, 1600, True, 250 + d), lens=lens)


@pytest.mark.parametrize("G", [1, 4, 8, 16, 24, 32])
def test_int4_decode_gqa_groups(K, G):
    run_int4(K, synth.DecodeCase("i4", 3, 2 * G, 2, 128, "bf16", 1, 700, True, 260 + G))


def test_int4_decode_workload(K):
    """The paged decode workload (B=64, H_q=32, H_kv=8, lengths 128 .. 8192) with an
    int4 cache, every (sequence, head)."""
    run_int4(K, synth.DECODE_PAGED)


def test_int4_bad_block_raises_flag(K):
    case = synth.DecodeCase("i4", 2, 4, 2, 64, "bf16", 20, 40, True, 270)
    inp = synth.int4_decode_inputs(case)
    table = inp["block_table"].copy()
    table[1, 0] = -7
    K.attn_decode_paged_int4(to_dev(inp["q"], "bf16"), u8(inp["k_pool"]), u8(inp["v_pool"]), to_dev_i32(table),
                             to_dev_i32(inp["lens"] + 1), f32(inp["k_scales"]), f32(inp["v_scales"]))
    assert K.attn_device_error_flags() & 2


# Lengths (after the append) around the 16-token blocks and the 64-token stages of
# the 4-bit decode, with every table entry past a sequence's last block outside
# the pool: a stage whose later blocks lie past the length must not read them.
STAGE_TAIL_LENS = np.array([0, 1, 15, 16, 17, 31, 32, 33, 46, 47, 48, 62, 63, 64, 78, 126, 127, 128, 190, 250],
                           dtype=np.int32)


@pytest.mark.parametrize("d", [64, 128])
def test_int4_decode_stage_tails_read_no_table_entry_past_the_length(K, d):
    run_int4(K, synth.DecodeCase("i4", len(STAGE_TAIL_LENS), 8, 2, d, "bf16", 0, 260, True, 280 + d),
             lens=STAGE_TAIL_LENS, poison=True)


@pytest.mark.parametrize("d", [64, 128])
def test_int8_decode_reads_no_table_entry_past_the_length(K, d):
    run_int8(K, synth.DecodeCase("i8", len(STAGE_TAIL_LENS), 8, 2, d, "f16", 0, 260, True, 290 + d),
             lens=STAGE_TAIL_LENS, poison=True)


@pytest.mark.parametrize("d", [64, 128])
def test_int8_decode_extreme_queries(K, d):
    run_int8(K, synth.DecodeCase("i8", 4, 8, 2, d, "bf16", 1, 300, True, 300 + d), edit=extreme_queries)


@pytest.mark.parametrize("d", [64, 128])
def test_int4_decode_extreme_queries(K, d):
    run_int4(K, synth.DecodeCase("i4", 4, 8, 2, d, "f16", 1, 300, True, 310 + d), edit=extreme_queries)


def test_int8_decode_two_head_groups_d64(K):
    """G = 24 at d = 64: two groups of query heads per KV head, the second partly filled."""
    run_int8(K, synth.DecodeCase("i8", 3, 48, 2, 64, "f16", 1, 700, True, 350))


def test_int4_decode_two_head_groups_d64(K):
    run_int4(K, synth.DecodeCase("i4", 3, 48, 2, 64, "f16", 1, 700, True, 351))
