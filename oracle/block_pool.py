"""A paged KV cache's block bookkeeping, and a serving simulation that compares
it with contiguous per-sequence reservations.

Test infrastructure only (see the package docstring).

What it models, cited by page title and section:

* "KV Cache:推理慢的真正原因", 工程优化手段 / 1 (PagedAttention): the cache is
  cut into fixed 16-token blocks; a block table maps a sequence's logical blocks
  to physical ones; blocks of a finished request are reused at once.  The same
  subsection states the motivation: a contiguous layout reserves max_len slots
  per sequence and wastes what is not used.
* "KV缓存与Flash注意力", 练习: the hard exercise (16-token blocks with a free
  list, blocks returned when a sequence finishes, 1,000 chat completions of
  different lengths, fragmentation against contiguous allocation) and the medium
  one (a prompt's cache filled once, then shared by the completions that branch
  from it).

Policy (the pages fix none of it; these are the readings this oracle defines):

* Free list: a stack.  Initially block 0 is on top, then 1, 2, ...; a freed
  block is pushed on top, so the most recently freed block is reused first.
* Reference counts: a block shared by forked sequences counts each holder.
  A block returns to the free list when its count reaches zero.
* Copy on write: before a sequence writes into its partially filled last block
  while another sequence still holds that block, it takes a fresh block, and
  the (old, new) pair is reported so the caller copies the contents.
* A reservation that cannot be met changes nothing and raises ``NoBlocks``.

Pins (tests/test_oracle_block_pool.py): hand-traced id sequences, the
holder-count invariant after random operation sequences, atomicity on
exhaustion and bad rows, and closed forms of the simulation's counters.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

BLOCK = 16


class NoBlocks(Exception):
    """The free list cannot meet a reservation."""


def blocks_for(n_tokens: int) -> int:
    """Blocks that hold n_tokens tokens: ceil(n / 16)."""
    return -(-n_tokens // BLOCK)


class FreeListPool:
    """num_blocks physical blocks, a free stack and a holder count per block."""

    def __init__(self, num_blocks: int):
        if num_blocks < 1:
            raise ValueError("num_blocks must be >= 1")
        self.num_blocks = num_blocks
        self.free: List[int] = list(range(num_blocks - 1, -1, -1))  # top of stack = end
        self.ref: List[int] = [0] * num_blocks

    def free_blocks(self) -> int:
        return len(self.free)

    def _check_row(self, row: Sequence[int], n_tokens: int, max_blocks: int) -> None:
        if n_tokens < 0 or blocks_for(n_tokens) > max_blocks or len(row) < max_blocks:
            raise ValueError("length outside the table row")
        for j in range(blocks_for(n_tokens)):
            b = row[j]
            if not (0 <= b < self.num_blocks) or self.ref[b] == 0:
                raise ValueError(f"row entry {j} ({b}) is not a held block")

    def reserve(self, row: List[int], cur_len: int, new_len: int, max_blocks: int) -> Optional[Tuple[int, int]]:
        """Make ``row`` cover new_len tokens of a sequence that holds cur_len.

        Returns the (old, new) block pair to copy when the partially filled last
        block was shared (copy on write), else None.
        """
        if new_len < cur_len:
            raise ValueError("new_len < cur_len")
        self._check_row(row, cur_len, max_blocks)
        if blocks_for(new_len) > max_blocks:
            raise ValueError("new_len exceeds the table row")
        last = blocks_for(cur_len) - 1
        cow = new_len > cur_len and cur_len % BLOCK != 0 and self.ref[row[last]] > 1
        need = blocks_for(new_len) - blocks_for(cur_len) + (1 if cow else 0)
        if need > len(self.free):
            raise NoBlocks(f"need {need} blocks, {len(self.free)} free")
        pair = None
        if cow:
            old = row[last]
            new = self.free.pop()
            self.ref[new] = 1
            self.ref[old] -= 1  # still > 0: another holder keeps it
            row[last] = new
            pair = (old, new)
        for j in range(blocks_for(cur_len), blocks_for(new_len)):
            b = self.free.pop()
            self.ref[b] = 1
            row[j] = b
        return pair

    def release(self, row: List[int], length: int, max_blocks: int) -> None:
        """Drop the sequence's hold on its blocks; blocks nobody holds go back on
        the free list in row order (the last one released is reused first)."""
        self._check_row(row, length, max_blocks)
        for j in range(blocks_for(length)):
            b = row[j]
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
            row[j] = -1

    def fork(self, src: Sequence[int], dst: List[int], length: int, max_blocks: int) -> None:
        """dst shares src's blocks for its first ``length`` tokens."""
        self._check_row(src, length, max_blocks)
        if len(dst) < max_blocks:
            raise ValueError("dst row too short")
        for j in range(blocks_for(length)):
            dst[j] = src[j]
            self.ref[src[j]] += 1


def simulate(prompts: Sequence[int], outputs: Sequence[int], memory_tokens: int, max_len: int,
             scheme: str) -> Dict[str, float]:
    """Serve every request (all arrive at step 0) with continuous batching.

    A request i holds prompt_i tokens once admitted and grows by one token per
    step until it holds prompt_i + output_i, then leaves and frees its memory.

    * ``"contiguous"``: admission reserves max_len slots out of memory_tokens;
      a sequence never needs more.
    * ``"paged"``: memory_tokens // 16 blocks.  Admission takes the blocks of the
      tokens the request holds, and only while at least W = ceil(1% of the
      blocks) would stay free.  A step that needs a block when none is free
      preempts the most recently admitted running request: its blocks are freed
      and it goes back to the front of the queue keeping the tokens it has (to
      be re-admitted holding them all).

    Each step: admit from the queue head while the request fits, then in
    admission order append one token to every running request (paged: taking a
    block when its length is a multiple of 16), retire finished ones, and
    count.  Counters: steps; token_steps = sum over steps of the tokens held;
    held_steps = sum of the slots held (contiguous: running * max_len; paged:
    16 * blocks held); preemptions; peak and summed running counts.
    """
    if scheme not in ("contiguous", "paged"):
        raise ValueError(scheme)
    R = len(prompts)
    total = [int(prompts[i]) + int(outputs[i]) for i in range(R)]
    if any(t > max_len for t in total) or any(int(o) < 1 for o in outputs) or any(int(p) < 1 for p in prompts):
        raise ValueError("every request needs prompt >= 1, output >= 1 and prompt + output <= max_len")
    held_tokens = [int(p) for p in prompts]  # tokens a request holds (kept across preemption)
    queue = list(range(R))  # front = index 0
    running: List[int] = []
    n_blocks = memory_tokens // BLOCK
    watermark = -(-n_blocks // 100)
    pool = FreeListPool(n_blocks) if scheme == "paged" else None
    rows: Dict[int, List[int]] = {}
    max_blocks = blocks_for(max_len)
    free_slots = memory_tokens
    stats = dict(steps=0, token_steps=0, held_steps=0, preemptions=0, peak_running=0, running_steps=0)

    while queue or running:
        # admission
        while queue:
            i = queue[0]
            if scheme == "contiguous":
                if free_slots < max_len:
                    break
                free_slots -= max_len
            else:
                need = blocks_for(held_tokens[i])
                if pool.free_blocks() - need < watermark:
                    break
                rows[i] = [-1] * max_blocks
                pool.reserve(rows[i], 0, held_tokens[i], max_blocks)
            queue.pop(0)
            running.append(i)
        if not running:
            raise RuntimeError("a request cannot be admitted into an empty memory")
        # one token for every running request, in admission order
        k = 0
        while k < len(running):
            i = running[k]
            L = held_tokens[i]
            if scheme == "paged" and L % BLOCK == 0:
                while pool.free_blocks() == 0:
                    victim = running.pop()
                    pool.release(rows.pop(victim), held_tokens[victim], max_blocks)
                    queue.insert(0, victim)
                    stats["preemptions"] += 1
                    if victim == i:
                        break
                if victim_gone(running, k, i):
                    continue
                pool.reserve(rows[i], L, L + 1, max_blocks)
            held_tokens[i] = L + 1
            if held_tokens[i] == total[i]:
                running.pop(k)
                if scheme == "contiguous":
                    free_slots += max_len
                else:
                    pool.release(rows.pop(i), held_tokens[i], max_blocks)
                continue
            k += 1
        # counters over the requests still holding memory after the step
        stats["steps"] += 1
        stats["token_steps"] += sum(held_tokens[i] for i in running)
        if scheme == "contiguous":
            stats["held_steps"] += len(running) * max_len
        else:
            stats["held_steps"] += BLOCK * (n_blocks - pool.free_blocks())
        stats["running_steps"] += len(running)
        stats["peak_running"] = max(stats["peak_running"], len(running))

    out: Dict[str, float] = dict(stats)
    out["utilization_held"] = stats["token_steps"] / stats["held_steps"] if stats["held_steps"] else 0.0
    out["utilization_budget"] = stats["token_steps"] / (stats["steps"] * memory_tokens)
    out["mean_running"] = stats["running_steps"] / stats["steps"]
    return out


def victim_gone(running: List[int], k: int, i: int) -> bool:
    """True when request i (expected at position k) was itself preempted."""
    return k >= len(running) or running[k] != i
