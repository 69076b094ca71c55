"""GPU side of the block pool: kv_copy_blocks copies whole blocks bit for bit, and
a serving loop over pool-managed block tables matches the oracle step by step.

The loop is the prefix-sharing exercise of "KV缓存与Flash注意力" (练习): one
prompt's cache is filled once, completions fork from it (sharing its blocks;
the partly filled last block is copied on first write), and every sequence then
decodes token by token.  Midway one sequence finishes and a new request takes
its place: its blocks are reused at once ("KV Cache:推理慢的真正原因",
工程优化手段 / 1) and still hold the old request's rows, which the decode must
not see.
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
    assert k.attn_device_error_flags() == 0
    return k


@pytest.mark.parametrize("np_dtype,d", [(np.uint8, 128), (np.int16, 128), (np.int16, 64), (np.float32, 32)])
def test_copy_blocks_bit_exact(K, np_dtype, d):
    print(f"[copy_blocks] {np.dtype(np_dtype).name} d={d}", flush=True)
    nb, H = 12, 4
    rng = np.random.default_rng(d)
    kp = rng.integers(0, 255, size=(nb, H, 16, d * np.dtype(np_dtype).itemsize), dtype=np.uint8).view(np_dtype)
    vp = rng.integers(0, 255, size=kp.shape[:3] + (d * np.dtype(np_dtype).itemsize,),
                      dtype=np.uint8).view(np_dtype)
    pairs = np.array([[0, 5], [3, 7], [11, 2], [6, 6]], dtype=np.int32)
    kd, vd = torch.from_numpy(kp.copy()).cuda(), torch.from_numpy(vp.copy()).cuda()
    K.kv_copy_blocks(kd, vd, to_dev_i32(pairs))
    torch.cuda.synchronize()
    assert K.attn_device_error_flags() == 0
    for s, t in pairs:
        kp[t] = kp[s]
        vp[t] = vp[s]
    assert kd.cpu().numpy().tobytes() == kp.tobytes() and vd.cpu().numpy().tobytes() == vp.tobytes()


def test_copy_blocks_bad_ids_are_skipped(K):
    print("[copy_blocks] bad ids", flush=True)
    nb, H, d = 6, 2, 64
    kp = np.arange(nb * H * 16 * d, dtype=np.int16).reshape(nb, H, 16, d)
    vp = kp[::-1].copy()
    kd, vd = torch.from_numpy(kp.copy()).cuda(), torch.from_numpy(vp.copy()).cuda()
    K.kv_copy_blocks(kd, vd, to_dev_i32(np.array([[0, 1], [-1, 3], [2, 99]], np.int32)))
    assert K.attn_device_error_flags() == 2
    kp[1], vp[1] = kp[0], vp[0]
    assert np.array_equal(kd.cpu().numpy(), kp) and np.array_equal(vd.cpu().numpy(), vp)
    K.kv_copy_blocks(kd, vd, to_dev_i32(np.zeros((0, 2), np.int32)))  # nothing to copy


def _rows(rng, shape, dtype):
    return synth.to_storage(rng.standard_normal(shape, dtype=np.float32), dtype)


@pytest.mark.parametrize("dtype,d,G", [("bf16", 128, 4), ("f16", 64, 2)])
def test_serving_loop_with_forks_and_reuse(K, dtype, d, G):
    from kv_cache_flashattention_attn_amd.block_pool import BlockPool
    print(f"[serving loop] {dtype} d={d} G={G}", flush=True)
    H_kv, C, Lp, T, mb = 2, 5, 37, 24, 6
    H_q, B = G * H_kv, C + 1
    scale = 1.0 / np.sqrt(d)
    max_len = mb * 16
    rng = synth.make_rng(900 + d)
    nb = 48
    pool = BlockPool(nb)
    table = np.full((B, mb), -1, np.int32)

    # device pools start as sentinels: K = 0 and V = 8192 in every slot
    kp = to_dev(synth.storage_fill((nb, H_kv, 16, d), synth.SENTINEL_K, dtype), dtype)
    vp = to_dev(synth.storage_fill((nb, H_kv, 16, d), synth.SENTINEL_V, dtype), dtype)
    # the oracle's view: each sequence's logical cache, contiguous
    ref = oracle.ContigCache(synth.storage_fill((B, H_kv, max_len, d), synth.SENTINEL_K, dtype),
                             synth.storage_fill((B, H_kv, max_len, d), synth.SENTINEL_V, dtype))

    # one pass over the prompt fills sequence 0's blocks
    kP, vP = _rows(rng, (1, H_kv, Lp, d), dtype), _rows(rng, (1, H_kv, Lp, d), dtype)
    pool.reserve(table[0], 0, Lp)
    K.kv_append(kp, vp, to_dev(kP, dtype), to_dev(vP, dtype), to_dev_i32(np.zeros(1, np.int32)),
                to_dev_i32(table[:1]))
    for b in range(B):
        ref.k[b, :, :Lp], ref.v[b, :, :Lp] = kP[0], vP[0]
    # the completions branch from it, sharing all three blocks
    for b in range(1, B):
        pool.fork(table[0], table[b], Lp)
    assert pool.holders(int(table[0, 2])) == B
    lens = np.full(B, Lp, np.int32)

    n_copies = 0
    for t in range(T):
        if t == T // 2:
            # sequence 2 finishes; a new request with a 20-token prompt takes its row
            pool.release(table[2], int(lens[2]))
            L2 = 20
            pool.reserve(table[2], 0, L2)
            k2, v2 = _rows(rng, (1, H_kv, L2, d), dtype), _rows(rng, (1, H_kv, L2, d), dtype)
            K.kv_append(kp, vp, to_dev(k2, dtype), to_dev(v2, dtype), to_dev_i32(np.zeros(1, np.int32)),
                        to_dev_i32(table[2:3]))
            ref.k[2], ref.v[2] = (synth.storage_fill((H_kv, max_len, d), synth.SENTINEL_K, dtype),
                                  synth.storage_fill((H_kv, max_len, d), synth.SENTINEL_V, dtype))
            ref.k[2, :, :L2], ref.v[2, :, :L2] = k2[0], v2[0]
            lens[2] = L2
        done, pairs = pool.reserve_batch(table, lens, lens + 1)
        assert done == B
        if len(pairs):
            K.kv_copy_blocks(kp, vp, to_dev_i32(pairs))
            n_copies += len(pairs)
        q = _rows(rng, (B, H_q, d), dtype)
        kn, vn = _rows(rng, (B, H_kv, 1, d), dtype), _rows(rng, (B, H_kv, 1, d), dtype)
        lens_d, table_d = to_dev_i32(lens), to_dev_i32(table)
        K.kv_append(kp, vp, to_dev(kn, dtype), to_dev(vn, dtype), lens_d, table_d)
        o, lse = K.attn_decode_paged(to_dev(q, dtype), kp, vp, table_d, to_dev_i32(lens + 1), scale=scale,
                                     return_lse=True)
        Oref, Lref = oracle.decode_step(ref, q, kn, vn, lens, scale, dtype)
        assert_close(values_of(o), Oref, dtype, what=f"O step {t}")
        assert_lse_close(lse.cpu().numpy().astype(np.float64), Lref, dtype, what=f"lse step {t}")
        lens += 1
    assert K.attn_device_error_flags() == 0
    # the first write after the fork copied the shared last block for all but its last holder
    assert n_copies == B - 1

    # every sequence's cache, gathered through its final row, is its logical cache bit for bit
    kb, vb = bits_of(kp), bits_of(vp)
    for b in range(B):
        L = int(lens[b])
        idx = [(int(table[b, p // 16]), p % 16) for p in range(L)]
        gk = np.stack([kb[i, :, s] for i, s in idx], axis=1)
        gv = np.stack([vb[i, :, s] for i, s in idx], axis=1)
        assert gk.tobytes() == np.ascontiguousarray(ref.k[b, :, :L]).tobytes(), f"K of sequence {b}"
        assert gv.tobytes() == np.ascontiguousarray(ref.v[b, :, :L]).tobytes(), f"V of sequence {b}"
    for b in range(B):
        pool.release(table[b], int(lens[b]))
    assert pool.free_blocks() == nb
