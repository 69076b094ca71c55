"""The native block pool (attn_block_pool_* in libattn) against the oracle's free
list, id for id, and the serving simulation against the oracle's, counter for
counter.  Host code only: no GPU is needed."""
import os

import numpy as np
import pytest

import oracle
import synth

klib = pytest.importorskip("kv_cache_flashattention_attn_amd")
if not os.path.exists(klib.lib_path):
    pytest.skip("libattn.so not built", allow_module_level=True)

from kv_cache_flashattention_attn_amd.block_pool import BlockPool, NoBlocks  # noqa: E402
from kv_cache_flashattention_attn_amd import serving_sim  # noqa: E402

MB = 8  # blocks per row


def _same_state(nat, ref):
    assert nat.free_blocks() == ref.free_blocks()
    assert [nat.holders(b) for b in range(ref.num_blocks)] == ref.ref


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_operations_match_the_oracle(seed):
    rng = np.random.default_rng(seed)
    nb = 48
    nat, ref = BlockPool(nb), oracle.FreeListPool(nb)
    live = {}  # id -> (native row, oracle row, length)
    nxt = 0
    for _ in range(2000):
        op = int(rng.integers(0, 4))
        if op == 0 or not live:
            L = int(rng.integers(1, 16 * MB + 1))
            rn, ro = np.full(MB, -1, np.int32), [-1] * MB
            try:
                ref.reserve(ro, 0, L, MB)
            except oracle.NoBlocks:
                with pytest.raises(NoBlocks):
                    nat.reserve(rn, 0, L)
                continue
            assert nat.reserve(rn, 0, L) is None
            live[nxt] = (rn, ro, L)
            nxt += 1
        else:
            k = list(live)[int(rng.integers(0, len(live)))]
            rn, ro, L = live[k]
            if op == 1:
                ref.release(ro, L, MB)
                nat.release(rn, L)
                del live[k]
            elif op == 2:
                new = min(16 * MB, L + int(rng.integers(0, 40)))
                try:
                    pair = ref.reserve(ro, L, new, MB)
                except oracle.NoBlocks:
                    with pytest.raises(NoBlocks):
                        nat.reserve(rn, L, new)
                else:
                    assert nat.reserve(rn, L, new) == pair
                    live[k] = (rn, ro, new)
            else:
                dn, do = np.full(MB, -1, np.int32), [-1] * MB
                ref.fork(ro, do, L, MB)
                nat.fork(rn, dn, L)
                live[nxt] = (dn, do, L)
                nxt += 1
        for rn, ro, L in live.values():
            assert rn.tolist() == ro
        _same_state(nat, ref)


def test_batch_reserve_equals_one_by_one():
    rng = np.random.default_rng(7)
    nb, B = 64, 10
    nat, ref = BlockPool(nb), oracle.FreeListPool(nb)
    table = np.full((B, MB), -1, np.int32)
    rows = [[-1] * MB for _ in range(B)]
    lens = rng.integers(1, 40, size=B).astype(np.int32)
    nat.reserve_batch(table, np.zeros(B, np.int32), lens)
    for b in range(B):
        ref.reserve(rows[b], 0, int(lens[b]), MB)
    # fork half of them onto the other half, then grow all: copies on write
    for b in range(0, B, 2):
        nat.release(table[b + 1], int(lens[b + 1]))
        ref.release(rows[b + 1], int(lens[b + 1]), MB)
        nat.fork(table[b], table[b + 1], int(lens[b]))
        ref.fork(rows[b], rows[b + 1], int(lens[b]), MB)
        lens[b + 1] = lens[b]
    new = lens + rng.integers(1, 20, size=B).astype(np.int32)
    done, pairs = nat.reserve_batch(table, lens, new)
    want = [p for b in range(B) if (p := ref.reserve(rows[b], int(lens[b]), int(new[b]), MB)) is not None]
    assert done == B
    assert pairs.tolist() == [list(p) for p in want]
    assert table.tolist() == rows
    _same_state(nat, ref)


def test_batch_reserve_stops_at_exhaustion():
    nat = BlockPool(5)
    table = np.full((3, MB), -1, np.int32)
    with pytest.raises(NoBlocks) as e:
        nat.reserve_batch(table, np.zeros(3, np.int32), np.array([32, 40, 16], np.int32))
    # rows 0 and 1 take 2 + 3 blocks; row 2 finds none and stays unassigned
    assert e.value.n_done == 2
    assert table[0].tolist() == [0, 1] + [-1] * (MB - 2)
    assert table[1].tolist() == [2, 3, 4] + [-1] * (MB - 3)
    assert table[2].tolist() == [-1] * MB and nat.free_blocks() == 0


def test_failed_calls_change_nothing():
    nat = BlockPool(4)
    row = np.full(MB, -1, np.int32)
    nat.reserve(row, 0, 33)
    snap = (row.copy(), nat.free_blocks(), [nat.holders(b) for b in range(4)])
    with pytest.raises(NoBlocks):
        nat.reserve(row, 33, 80)
    with pytest.raises(klib.AttnError):
        nat.reserve(row, 33, 16 * MB + 1)
    with pytest.raises(klib.AttnError):
        nat.reserve(row, 40, 30)
    bad = row.copy()
    bad[1] = 9
    with pytest.raises(klib.AttnError):
        nat.release(bad, 33)
    with pytest.raises(klib.AttnError):
        nat.fork(np.full(MB, -1, np.int32), np.full(MB, -1, np.int32), 1)
    assert (row.tolist(), nat.free_blocks(), [nat.holders(b) for b in range(4)]) == \
        (snap[0].tolist(), snap[1], snap[2])
    assert nat.holders(4) == -1 and nat.holders(-1) == -1
    with pytest.raises(klib.AttnError):
        BlockPool(0)


@pytest.mark.parametrize("scheme", ["contiguous", "paged"])
def test_simulation_matches_the_oracle(scheme):
    c = synth.CHAT_SIM
    prompts, outputs = synth.chat_requests(c)
    got = serving_sim.simulate(prompts, outputs, c.memory_tokens, c.max_len, scheme)
    want = oracle.simulate(prompts.tolist(), outputs.tolist(), c.memory_tokens, c.max_len, scheme)
    assert got == want


@pytest.mark.parametrize("memory_tokens", [48, 64 * 16, 4096])
def test_small_simulations_match_the_oracle(memory_tokens):
    rng = np.random.default_rng(memory_tokens)
    prompts = rng.integers(1, 30, size=40).tolist()
    outputs = rng.integers(1, 18, size=40).tolist()
    for scheme in ("contiguous", "paged"):
        got = serving_sim.simulate(prompts, outputs, memory_tokens, 48, scheme)
        want = oracle.simulate(prompts, outputs, memory_tokens, 48, scheme)
        assert got == want


def test_paged_memory_claim_on_the_chat_workload():
    c = synth.CHAT_SIM
    prompts, outputs = synth.chat_requests(c)
    con = serving_sim.simulate(prompts, outputs, c.memory_tokens, c.max_len, "contiguous")
    pag = serving_sim.simulate(prompts, outputs, c.memory_tokens, c.max_len, "paged")
    # utilisation rises from well under half to over 90%, and the same memory
    # serves about twice as many requests at once
    assert 0.2 <= con["utilization_held"] <= 0.45
    assert pag["utilization_held"] >= 0.9
    assert 2.0 <= pag["mean_running"] / con["mean_running"] <= 3.0
