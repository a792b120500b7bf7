"""Pins of the oracle's allocator replay (oracle/allocator_replay.py) against hand-worked
step traces and the page's own statements (spindle, "Paging"), and planted mistakes in
copies of it that the pins must catch."""

import os
import sys
import types

import pytest

from oracle import allocator_replay as ar

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def check_single_request(m):
    # prompt 16, one generated token: holds 17 tokens for one step
    c = m.replay(m.CONTIGUOUS, [16], [1], 192, 8192)
    assert (c.steps, c.peak_slots, c.slots_trace, c.tokens_trace) == (1, 208, [208], [17])
    assert c.mean_utilisation == pytest.approx(17 / 208)
    p = m.replay(m.PAGED, [16], [1], 192, 8192)
    assert (p.steps, p.peak_slots, p.slots_trace, p.tokens_trace) == (1, 32, [32], [17])
    assert p.mean_utilisation == pytest.approx(17 / 32)


def check_stop_at_20_of_192(m):
    """The page's example: a contiguous buffer reserved for 192 new tokens stays reserved
    in full (here prompt 4 + 192) while its request produces only 20; the pool holds only
    what the request has written."""
    c = m.replay(m.CONTIGUOUS, [4], [20], 192, 8192)
    assert c.slots_trace == [196] * 20
    assert c.tokens_trace == list(range(5, 25))
    p = m.replay(m.PAGED, [4], [20], 192, 8192)
    assert p.tokens_trace == list(range(5, 25))
    assert p.slots_trace == [16] * 12 + [32] * 8   # 5..16 tokens -> 1 block, 17..24 -> 2
    assert p.peak_slots == 32


def check_waste_bound(m):
    """Pool: slots - tokens < block_size per running request, every step."""
    from workloads.synth import allocator_replay_requests
    pr, gn, kw = allocator_replay_requests(3)
    p = m.replay(m.PAGED, pr, gn, **kw)
    assert p.steps > 0
    for s, t, n in zip(p.slots_trace, p.tokens_trace, p.running_trace):
        assert 0 <= s - t < kw["block_size"] * n
    c = m.replay(m.CONTIGUOUS, pr, gn, **kw)
    assert all(s >= t for s, t in zip(c.slots_trace, c.tokens_trace))


def check_serialised(m):
    # each reservation 16 + 20 = 36 slots; 64 slots hold one at a time, while the pool
    # (4 blocks) holds both: 17..23 tokens are 2 blocks each
    c = m.replay(m.CONTIGUOUS, [16, 16], [5, 7], 20, 64)
    assert c.steps == 12
    assert c.running_trace == [1] * 12
    assert c.slots_trace == [36] * 12
    assert c.tokens_trace == list(range(17, 22)) + list(range(17, 24))
    p = m.replay(m.PAGED, [16, 16], [5, 7], 20, 64)
    assert p.steps == 7 and p.preemptions == 0
    assert p.running_trace == [2] * 5 + [1] * 2
    assert p.slots_trace == [64] * 5 + [32] * 2
    assert p.tokens_trace == [34, 36, 38, 40, 42, 22, 23]


def check_first_fit_and_merge(m):
    """Three 36-slot reservations fill [0, 108) of 128 slots; the fourth waits for the
    first to leave and takes its hole (first fit); a 72-slot request then needs the holes
    [0, 36) and [36, 72) merged."""
    c = m.replay(m.CONTIGUOUS, [16, 16, 16, 16, 52], [2, 4, 6, 3, 1], 20, 128)
    # r0 leaves after step 2, r3 takes [0, 36) at step 3; r1 leaves after step 4 and r3
    # after step 5, so [0, 72) is one run at step 6, where r4 runs its single step
    assert c.running_trace == [3, 3, 3, 3, 2, 2]
    assert c.steps == 6
    assert c.slots_trace == [108, 108, 108, 108, 72, 108]
    # 3 x 17; 3 x 18; r3 17 + 2 x 19; 20 + 20 + 18; 21 + 19; r4 53 + r2 22
    assert c.tokens_trace == [51, 54, 55, 58, 40, 75]


def check_preemption_by_hand(m):
    """Pool of 3 blocks: r0 (prompt 15, gen 20) outgrows it while r1 (prompt 15, gen 5)
    is preempted every second step, then runs after r0 leaves."""
    p = m.replay(m.PAGED, [15, 15], [20, 5], 20, 48)
    assert p.steps == 25
    assert p.preemptions == 9
    assert p.slots_trace[:17] == [32] + [48 if t % 2 == 1 else 32 for t in range(2, 18)]
    assert p.slots_trace[17:] == [48, 48, 48, 16, 32, 32, 32, 32]
    tokens = [32] + [(15 + t) + (16 if t % 2 == 1 else 0) for t in range(2, 18)]
    assert p.tokens_trace[:17] == tokens
    assert p.tokens_trace[17:] == [33, 34, 35, 16, 17, 18, 19, 20]
    assert p.peak_slots == 48


def check_no_overtaking(m):
    """FIFO without overtaking: r2 (36 slots) fits beside r0 but waits behind r1 (120)."""
    c = m.replay(m.CONTIGUOUS, [16, 100, 16], [10, 1, 1], 20, 128)
    assert c.steps == 12
    assert c.running_trace == [1] * 12
    assert c.slots_trace == [36] * 10 + [120, 36]


def check_first_fit_lowest_address(m):
    """The arena hands out the lowest hole that fits, not the tightest, and merges."""
    a = m._Contiguous(100)
    assert [a.alloc(40), a.alloc(30), a.alloc(30)] == [0, 40, 70]
    a.release(0, 40)
    a.release(70, 30)
    assert a.alloc(25) == 0          # lowest hole [0, 40), though [70, 100) is tighter
    a.release(40, 30)                # [25, 40) + [40, 70) + [70, 100) merge
    assert a.free == [(25, 75)]
    assert a.alloc(75) == 25 and a.alloc(1) is None


def check_admission_counts_first_token(m):
    """A 16-token prompt plus its first token needs 2 blocks: with 3 blocks the second
    request waits a step."""
    p = m.replay(m.PAGED, [16, 16], [1, 1], 20, 48)
    assert (p.steps, p.running_trace, p.slots_trace, p.tokens_trace) == \
        (2, [1, 1], [32, 32], [17, 17])


def check_preempted_returns_to_front(m):
    """r1 is preempted while r2 (2 blocks) waits; r1 must be readmitted first, so the
    oscillation of the 3-block case still shows (48 slots on odd steps)."""
    p = m.replay(m.PAGED, [15, 15, 16], [20, 5, 1], 20, 48)
    assert p.steps == 25 and p.preemptions == 9
    assert p.slots_trace[:4] == [32, 32, 48, 32]
    assert p.slots_trace[20:] == [48, 32, 32, 32, 32]   # r1 + r2 at step 21, then r1
    assert p.tokens_trace[20:] == [33, 17, 18, 19, 20]


def check_never_fit_rejected(m):
    with pytest.raises(ValueError):
        m.replay(m.CONTIGUOUS, [100], [1], 192, 256)
    with pytest.raises(ValueError):
        m.replay(m.PAGED, [15], [20], 20, 32)


CHECKS = [check_single_request, check_stop_at_20_of_192, check_waste_bound, check_serialised,
          check_first_fit_and_merge, check_preemption_by_hand, check_no_overtaking,
          check_first_fit_lowest_address, check_admission_counts_first_token,
          check_preempted_returns_to_front, check_never_fit_rejected]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_oracle_replay_pin(check):
    check(ar)


def _mutant(old, new):
    src = open(os.path.join(ORACLE_DIR, "allocator_replay.py")).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    name = "oracle.mutant_allocator_replay"
    mod = types.ModuleType(name)
    mod.__package__ = "oracle"
    sys.modules[name] = mod  # dataclasses look their module up
    try:
        exec(compile(src.replace(old, new, 1), "allocator_replay.py", "exec"), mod.__dict__)
    finally:
        del sys.modules[name]
    return mod


MUTANTS = {
    "no merge of freed runs": ("merged[-1] = (merged[-1][0], merged[-1][1] + n)",
                               "merged.append((s, n))"),
    "best fit instead of first fit": ("for k, (start, length) in enumerate(self.free):",
                                      "for k, (start, length) in sorted(enumerate(self.free), "
                                      "key=lambda x: x[1][1]):"),
    "admission overtakes": ("                if start is None:\n                    break",
                            "                if start is None:\n                    waiting.rotate(-1)\n"
                            "                    break"),
    "reserve prompt + gen": ("reserve = [p + max_new_tokens for p in prompt]",
                             "reserve = [p + g for p, g in zip(prompt, gen)]"),
    "paged admits without the first token": ("blocks_for(prompt[r] + 1)", "blocks_for(prompt[r])"),
    "preempt the oldest": ("victim = running.pop()", "victim = running.pop(0)"),
    "preempted request to the back": ("waiting.appendleft(victim)", "waiting.append(victim)"),
    "stats after leaving": ("        for r in [r for r in running if length[r] == prompt[r] + gen[r]]:",
                            "        for r in []:"),
    "leaves one token early": ("length[r] == prompt[r] + gen[r]]", "length[r] >= prompt[r] + gen[r] - 1]"),
    "utilisation as slots over tokens": ("util_sum += tokens / slots if slots else 0.0",
                                         "util_sum += slots / tokens if tokens else 0.0"),
    "new block one token late": ("if length[r] == len(pool.table(sid)) * block_size:",
                                 "if length[r] == len(pool.table(sid)) * block_size + 1:"),
}


def _caught(mod):
    for chk in CHECKS:
        try:
            chk(mod)
        except Exception:  # AssertionError, or the mutant crashing or stalling outright
            return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_replay_mutant_is_caught(name):
    old, new = MUTANTS[name]
    assert _caught(_mutant(old, new)), f"{name} survived"
