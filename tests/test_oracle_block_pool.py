"""Pins of the block-pool oracle (oracle/block_pool.py) against hand traces,
invariants and closed forms."""
import numpy as np
import pytest

from oracle.block_pool import FreeListPool, NoBlocks, blocks_for, simulate
import synth


def test_free_list_hand_trace():
    p = FreeListPool(4)
    A, B, C = [-1] * 4, [-1] * 4, [-1] * 4
    assert p.reserve(A, 0, 20, 4) is None and A[:2] == [0, 1]
    assert p.reserve(B, 0, 5, 4) is None and B[:1] == [2]
    p.release(A, 20, 4)  # pushes 0 then 1: 1 is on top
    assert A == [-1] * 4 and p.free_blocks() == 3
    p.reserve(C, 0, 17, 4)
    assert C[:2] == [1, 0]
    p.reserve(C, 17, 40, 4)
    assert C[:3] == [1, 0, 3] and p.free_blocks() == 0
    assert p.reserve(B, 5, 16, 4) is None  # fills block 2, no new block
    with pytest.raises(NoBlocks):
        p.reserve(B, 16, 17, 4)
    assert B == [2, -1, -1, -1]


def test_fork_and_copy_on_write():
    p = FreeListPool(8)
    A, F, G = [-1] * 4, [-1] * 4, [-1] * 4
    p.reserve(A, 0, 20, 4)  # [0, 1]
    p.fork(A, F, 20, 4)
    assert F[:2] == [0, 1] and p.ref[0] == 2 and p.ref[1] == 2
    assert p.reserve(F, 20, 21, 4) == (1, 2)  # last block shared and partly filled: copy it
    assert F[:2] == [0, 2] and p.ref[1] == 1 and p.ref[2] == 1
    assert p.reserve(A, 20, 21, 4) is None and A[:2] == [0, 1]  # A alone holds block 1 now
    p.release(A, 21, 4)  # block 0 still held by F, block 1 freed
    assert p.ref[0] == 1 and p.ref[1] == 0 and p.free[-1] == 1
    # a fork at a block boundary shares whole blocks only: no copy
    p.fork(F, G, 16, 4)
    assert p.reserve(G, 16, 17, 4) is None and G[:2] == [0, 1]
    assert p.ref[0] == 2


def test_failed_calls_change_nothing():
    p = FreeListPool(3)
    A = [-1] * 4
    p.reserve(A, 0, 33, 4)
    snap = (list(p.free), list(p.ref), list(A))
    with pytest.raises(NoBlocks):
        p.reserve(A, 33, 49, 4)
    with pytest.raises(ValueError):
        p.reserve(A, 33, 65, 4)  # beyond the row
    bad = [0, 7, -1, -1]
    with pytest.raises(ValueError):
        p.release(bad, 20, 4)  # 7 is no block
    with pytest.raises(ValueError):
        p.release([-1] * 4, 1, 4)  # an unassigned entry
    assert (list(p.free), list(p.ref), list(A)) == snap


def _check_invariants(p, rows):
    held = {}
    for row, L in rows.values():
        for j in range(blocks_for(L)):
            held[row[j]] = held.get(row[j], 0) + 1
    assert len(set(p.free)) == len(p.free)
    for b in range(p.num_blocks):
        assert p.ref[b] == held.get(b, 0)
        assert (b in p.free) == (p.ref[b] == 0)


def test_random_operations_keep_holder_counts():
    rng = np.random.default_rng(3)
    p = FreeListPool(40)
    rows = {}  # id -> (row, length)
    nxt = 0
    for _ in range(3000):
        op = rng.integers(0, 4)
        if op == 0 or not rows:
            row, L = [-1] * 8, int(rng.integers(1, 100))
            try:
                p.reserve(row, 0, L, 8)
            except NoBlocks:
                continue
            rows[nxt] = (row, L)
            nxt += 1
        else:
            k = list(rows)[int(rng.integers(0, len(rows)))]
            row, L = rows[k]
            if op == 1:
                p.release(row, L, 8)
                del rows[k]
            elif op == 2:
                new = min(128, L + int(rng.integers(1, 40)))
                try:
                    p.reserve(row, L, new, 8)
                    rows[k] = (row, new)
                except NoBlocks:
                    pass
            else:
                dst = [-1] * 8
                p.fork(row, dst, L, 8)
                rows[nxt] = (dst, L)
                nxt += 1
        _check_invariants(p, rows)


def test_random_partial_forks_copy_on_write():
    rng = np.random.default_rng(5)
    p = FreeListPool(64)
    rows = {}
    row = [-1] * 8
    p.reserve(row, 0, 37, 8)
    rows[0] = (row, 37)
    copies = 0
    for k in range(1, 20):
        src, L = rows[int(rng.integers(0, len(rows)))]
        dst = [-1] * 8
        p.fork(src, dst, L, 8)
        rows[k] = (dst, L)
        new = min(128, L + int(rng.integers(1, 30)))
        pair = p.reserve(dst, L, new, 8)
        if L % 16:
            assert pair is not None and dst[blocks_for(L) - 1] == pair[1]
            copies += 1
        rows[k] = (dst, new)
        _check_invariants(p, rows)
    assert copies > 0


def _lifetime_tokens(prompts, outputs):
    # a request holds p + 1, ..., p + n - 1 tokens at the ends of the steps it
    # runs without finishing, whatever the schedule
    return sum((n - 1) * p + n * (n - 1) // 2 for p, n in zip(prompts, outputs))


@pytest.mark.parametrize("scheme", ["contiguous", "paged"])
def test_simulation_single_request_closed_form(scheme):
    p, n, max_len = 37, 50, 128
    r = simulate([p], [n], max_len, max_len, scheme)
    assert r["steps"] == n and r["preemptions"] == 0 and r["peak_running"] == 1
    assert r["token_steps"] == (n - 1) * p + n * (n - 1) // 2
    if scheme == "contiguous":
        assert r["held_steps"] == (n - 1) * max_len
    else:
        assert r["held_steps"] == sum(16 * (-(-(p + t) // 16)) for t in range(1, n))


@pytest.mark.parametrize("scheme", ["contiguous", "paged"])
def test_simulation_ample_memory(scheme):
    prompts, outputs = [5, 16, 33, 100], [1, 20, 7, 64]
    r = simulate(prompts, outputs, 4 * 256 * 4, 256, scheme)
    assert r["steps"] == max(outputs) and r["preemptions"] == 0 and r["peak_running"] == 3
    assert r["token_steps"] == _lifetime_tokens(prompts, outputs)
    assert r["running_steps"] == sum(n - 1 for n in outputs)


def test_simulation_preemption_hand_trace():
    # 3 blocks, watermark 1: both requests admitted, the second is preempted at
    # its first block boundary and finishes after the first.
    r = simulate([15, 15], [10, 10], 48, 64, "paged")
    assert r["preemptions"] == 1 and r["steps"] == 19
    assert r["token_steps"] == 32 + 2 * sum(range(17, 25))
    assert r["held_steps"] == 32 * 17


def test_simulation_workload_counters_are_schedule_free():
    c = synth.CHAT_SIM
    prompts, outputs = synth.chat_requests(c)
    prompts, outputs = prompts[:200].tolist(), outputs[:200].tolist()
    rc = simulate(prompts, outputs, c.memory_tokens // 4, c.max_len, "contiguous")
    rp = simulate(prompts, outputs, c.memory_tokens // 4, c.max_len, "paged")
    for r in (rc, rp):
        assert r["token_steps"] == _lifetime_tokens(prompts, outputs)
        assert r["running_steps"] == sum(n - 1 for n in outputs)
    assert rc["peak_running"] == c.memory_tokens // 4 // c.max_len
    assert rp["preemptions"] > 0  # the paged run is memory-bound here


def test_chat_lengths_recipe():
    c = synth.CHAT_SIM
    prompts, outputs = synth.chat_requests(c)
    assert len(prompts) == len(outputs) == 1000
    assert prompts.min() >= 16 and prompts.max() <= 1024 and outputs.min() >= 16 and outputs.max() <= 1024
    assert (prompts + outputs).max() <= c.max_len
