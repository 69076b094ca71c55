"""Serving simulation over the native block pool: how much of the KV-cache memory
holds tokens when requests reserve contiguous max_len runs, and when they take
16-token blocks as they grow.

The comparison is the one of "KV Cache:推理慢的真正原因" (工程优化手段 / 1: a
contiguous cache reserves max_len per sequence and wastes what is unused; paged
blocks lift memory use and the number of concurrent requests), run as the
exercise of "KV缓存与Flash注意力" (练习: 1,000 chat completions of different
lengths, blocks from a free list returned when a sequence finishes).

Schedule (continuous batching; every request arrives at step 0):

* each step first admits requests from the head of the queue while they fit,
  then gives every running request one more token in admission order, retires
  the finished ones and counts what is held;
* contiguous: admission reserves max_len slots, which always suffice;
* paged: memory_tokens // 16 blocks in a BlockPool.  Admission takes the
  blocks of the tokens a request holds while at least ceil(1% of the blocks)
  stay free.  A request whose length is a multiple of 16 takes a block before
  its next token; if none is free, the most recently admitted running request
  is preempted (its blocks go back, it returns to the queue front keeping its
  tokens) until one is, or until the request itself was the one preempted.

Counters: steps, token_steps (tokens held summed over steps), held_steps
(slots held: running * max_len, or 16 * blocks held), preemptions, running
counts; utilisation = token_steps / held_steps and token_steps / (steps *
memory_tokens).
"""
from __future__ import annotations

from collections import deque
from typing import Dict, Sequence

import numpy as np

from .block_pool import BlockPool

BLOCK = 16


def _ceil_blocks(n: int) -> int:
    return (n + BLOCK - 1) // BLOCK


class _Contiguous:
    def __init__(self, memory_tokens: int, max_len: int):
        self.free, self.max_len = memory_tokens, max_len

    def admit(self, i: int, tokens: int) -> bool:
        if self.free < self.max_len:
            return False
        self.free -= self.max_len
        return True

    def grow(self, i: int, tokens: int) -> bool:  # room is reserved up front
        return True

    def retire(self, i: int, tokens: int) -> None:
        self.free += self.max_len

    def held_slots(self, n_running: int) -> int:
        return n_running * self.max_len


class _Paged:
    def __init__(self, memory_tokens: int, max_len: int, n_requests: int):
        self.n_blocks = memory_tokens // BLOCK
        self.pool = BlockPool(self.n_blocks)
        self.watermark = -(-self.n_blocks // 100)
        self.table = np.full((n_requests, _ceil_blocks(max_len)), -1, dtype=np.int32)

    def admit(self, i: int, tokens: int) -> bool:
        if self.pool.free_blocks() - _ceil_blocks(tokens) < self.watermark:
            return False
        self.pool.reserve(self.table[i], 0, tokens)
        return True

    def grow(self, i: int, tokens: int) -> bool:
        """Room for token number tokens + 1; False when no block is free."""
        if tokens % BLOCK:
            return True
        if self.pool.free_blocks() == 0:
            return False
        self.pool.reserve(self.table[i], tokens, tokens + 1)
        return True

    def retire(self, i: int, tokens: int) -> None:
        self.pool.release(self.table[i], tokens)

    def held_slots(self, n_running: int) -> int:
        return BLOCK * (self.n_blocks - self.pool.free_blocks())


def simulate(prompts: Sequence[int], outputs: Sequence[int], memory_tokens: int, max_len: int,
             scheme: str) -> Dict[str, float]:
    prompts = [int(x) for x in prompts]
    outputs = [int(x) for x in outputs]
    n = len(prompts)
    if len(outputs) != n:
        raise ValueError("prompts and outputs differ in length")
    if any(p < 1 or o < 1 or p + o > max_len for p, o in zip(prompts, outputs)):
        raise ValueError("every request needs prompt >= 1, output >= 1 and prompt + output <= max_len")
    if scheme == "contiguous":
        mem = _Contiguous(memory_tokens, max_len)
    elif scheme == "paged":
        mem = _Paged(memory_tokens, max_len, n)
    else:
        raise ValueError(scheme)

    goal = [p + o for p, o in zip(prompts, outputs)]
    tokens = list(prompts)
    waiting = deque(range(n))
    running: list = []
    steps = token_steps = held_steps = preemptions = peak = running_steps = 0

    while waiting or running:
        while waiting and mem.admit(waiting[0], tokens[waiting[0]]):
            running.append(waiting.popleft())
        if not running:
            raise RuntimeError("a request does not fit into empty memory")
        survivors = []
        pos = 0
        while pos < len(running):
            i = running[pos]
            preempted_self = False
            while not mem.grow(i, tokens[i]):
                victim = running.pop()
                mem.retire(victim, tokens[victim])
                waiting.appendleft(victim)
                preemptions += 1
                if victim == i:
                    preempted_self = True
                    break
            if preempted_self:
                break  # i was the last running request
            tokens[i] += 1
            if tokens[i] == goal[i]:
                mem.retire(i, tokens[i])
            else:
                survivors.append(i)
            pos += 1
        running = survivors
        steps += 1
        running_steps += len(running)
        peak = max(peak, len(running))
        token_steps += sum(tokens[i] for i in running)
        held_steps += mem.held_slots(len(running))

    return {
        "steps": steps, "token_steps": token_steps, "held_steps": held_steps, "preemptions": preemptions,
        "peak_running": peak, "running_steps": running_steps,
        "utilization_held": token_steps / held_steps if held_steps else 0.0,
        "utilization_budget": token_steps / (steps * memory_tokens),
        "mean_running": running_steps / steps,
    }
