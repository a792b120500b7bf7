"""Plain-Python replay of requests through two KV allocators (test infrastructure only).

spindle, section "Paging", compares a contiguous per-sequence buffer with the
block pool on 64 requests, 8192 token slots and 16-token blocks, and reports
peak slots held, mean slot utilisation and steps to drain.  It states why the
two differ: a contiguous buffer must be sized at admission to prompt +
max_new_tokens (the only bound known then) and is held whole for the request's
lifetime, while the pool hands out fixed-size blocks as tokens arrive, so a
sequence wastes at most its final partial block.  The page does not give its
workload or step model; the plainest reading, shared by both allocators:

* requests wait in a FIFO queue and are admitted in order at the start of a
  step while memory allows; the first one that does not fit stops admission
  (no overtaking);
* a request admitted in a step prefills its prompt and produces its first
  token in that step, holding prompt + 1 tokens afterwards; every later step
  adds one token; a request with generation length g leaves at the end of the
  step in which it holds prompt + g tokens;
* contiguous: admission needs a free run of prompt + max_new slots (first fit,
  lowest address), held until the request leaves; freed runs merge with their
  neighbours;
* paged: admission needs the blocks covering prompt + 1 tokens; a running
  request whose next token starts a new block takes one before writing it;
  when the pool is empty the most recently admitted running request is
  preempted (its blocks freed, its progress dropped, and it returns to the
  front of the queue) until a block is free, or until the request itself was
  the one preempted;
* per step, after the writes and before the leaving requests release memory:
  slots held = reserved slots (contiguous) or blocks x block size (paged) over
  running requests, tokens held = their cached tokens; peak slots held is the
  maximum over steps, mean slot utilisation the mean over steps of tokens /
  slots, and steps to drain the number of steps until no request remains.
"""

from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field

from .block_pool import BlockPool

CONTIGUOUS = 0
PAGED = 1


@dataclass
class ReplayResult:
    peak_slots: int
    mean_utilisation: float
    steps: int
    preemptions: int
    slots_trace: list = field(default_factory=list)
    tokens_trace: list = field(default_factory=list)
    running_trace: list = field(default_factory=list)


class _Contiguous:
    """First-fit allocator over one linear range of token slots."""

    def __init__(self, total):
        self.free = [(0, total)]  # (start, length), sorted, never adjacent

    def alloc(self, size):
        for k, (start, length) in enumerate(self.free):
            if length >= size:
                if length == size:
                    del self.free[k]
                else:
                    self.free[k] = (start + size, length - size)
                return start
        return None

    def release(self, start, size):
        self.free.append((start, size))
        self.free.sort()
        merged = []
        for s, n in self.free:
            if merged and merged[-1][0] + merged[-1][1] == s:
                merged[-1] = (merged[-1][0], merged[-1][1] + n)
            else:
                merged.append((s, n))
        self.free = merged


def replay(policy, prompt_lens, gen_lens, max_new_tokens, total_slots, block_size=16):
    """Run the requests to completion; returns a ReplayResult with per-step traces."""
    n_req = len(prompt_lens)
    prompt = [int(x) for x in prompt_lens]
    gen = [int(x) for x in gen_lens]
    if any(g < 1 or g > max_new_tokens for g in gen) or any(p < 0 for p in prompt):
        raise ValueError("need 1 <= gen <= max_new_tokens and prompt >= 0")
    if total_slots % block_size:
        raise ValueError("total_slots must be a multiple of block_size")
    # a request that cannot fit an empty pool on its own would never finish
    for p, g in zip(prompt, gen):
        if (policy == CONTIGUOUS and p + max_new_tokens > total_slots) or \
                (policy == PAGED and -(-(p + g) // block_size) > total_slots // block_size):
            raise ValueError("a request does not fit in an empty pool")
    waiting = deque(range(n_req))
    running = []   # request ids in admission order
    length = [0] * n_req
    if policy == CONTIGUOUS:
        arena = _Contiguous(total_slots)
        where = {}
        reserve = [p + max_new_tokens for p in prompt]
    elif policy == PAGED:
        pool = BlockPool(total_slots // block_size, block_size)
        seq_of = {}
    else:
        raise ValueError("unknown policy")

    def blocks_for(tokens):
        return -(-tokens // block_size)

    result = ReplayResult(0, 0.0, 0, 0)
    util_sum = 0.0
    # The oldest running request is never preempted (it would have to hold the whole
    # pool) and gains a token every step after its admission, so the replay ends within
    # sum(gen + 1) steps plus one admission step per request; past that it is stuck.
    step_bound = 4 * (sum(g + 1 for g in gen) + n_req) + 16
    while waiting or running:
        result.steps += 1
        if result.steps > step_bound:
            raise RuntimeError("replay does not make progress")
        admitted = set()
        while waiting:
            r = waiting[0]
            if policy == CONTIGUOUS:
                start = arena.alloc(reserve[r])
                if start is None:
                    break
                where[r] = start
            else:
                if pool.num_free() < blocks_for(prompt[r] + 1):
                    break
                sid = pool.add_sequence()
                pool.prepare_write(sid, 0, prompt[r] + 1)
                seq_of[r] = sid
            waiting.popleft()
            running.append(r)
            admitted.add(r)
            length[r] = prompt[r] + 1
        if not running:
            raise ValueError("a request does not fit in an empty pool")
        k = 0
        while k < len(running):
            r = running[k]
            if r in admitted:
                k += 1
                continue
            if policy == PAGED:
                sid = seq_of[r]
                if length[r] == len(pool.table(sid)) * block_size:
                    preempted_self = False
                    while pool.num_free() == 0:
                        victim = running.pop()
                        pool.free_sequence(seq_of.pop(victim))
                        length[victim] = 0
                        admitted.discard(victim)
                        waiting.appendleft(victim)
                        result.preemptions += 1
                        if victim == r:
                            preempted_self = True
                            break
                    if preempted_self:
                        continue  # r left running; running[k] is now past the end
                    pool.prepare_write(sid, length[r], 1)
            length[r] += 1
            k += 1
        if policy == CONTIGUOUS:
            slots = sum(reserve[r] for r in running)
        else:
            slots = sum(len(pool.table(seq_of[r])) * block_size for r in running)
        tokens = sum(length[r] for r in running)
        result.slots_trace.append(slots)
        result.tokens_trace.append(tokens)
        result.running_trace.append(len(running))
        result.peak_slots = max(result.peak_slots, slots)
        util_sum += tokens / slots if slots else 0.0
        for r in [r for r in running if length[r] == prompt[r] + gen[r]]:
            running.remove(r)
            if policy == CONTIGUOUS:
                arena.release(where.pop(r), reserve[r])
            else:
                pool.free_sequence(seq_of.pop(r))
    result.mean_utilisation = util_sum / result.steps if result.steps else 0.0
    return result
