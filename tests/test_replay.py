"""The native allocator replay (pkv_replay_allocator) against the oracle's replay, step
trace by step trace (host code only: no GPU)."""

import numpy as np
import pytest

from libpkv_util import ensure_built
from oracle import allocator_replay as ar
from workloads.synth import allocator_replay_requests


@pytest.fixture(scope="module", autouse=True)
def _built():
    ensure_built()


def _native():
    from paged_kv_cache_200_amd import replay
    return replay


def _same(policy, prompts, gens, max_new, total, block=16):
    want = ar.replay(policy, prompts, gens, max_new, total, block)
    got = _native().replay_allocator(policy, prompts, gens, max_new, total, block, trace=True)
    assert got["steps"] == want.steps
    assert got["preemptions"] == want.preemptions
    assert got["peak_slots"] == want.peak_slots
    assert got["slots_trace"] == want.slots_trace
    assert got["tokens_trace"] == want.tokens_trace
    assert got["running_trace"] == want.running_trace
    assert got["mean_utilisation"] == pytest.approx(want.mean_utilisation, rel=1e-12)
    return got


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("policy", [ar.CONTIGUOUS, ar.PAGED])
def test_workload_traces_match(seed, policy):
    p, g, kw = allocator_replay_requests(seed)
    _same(policy, p, g, kw["max_new_tokens"], kw["total_slots"], kw["block_size"])


@pytest.mark.parametrize("seed", range(12))
def test_random_small_pools_match(seed):
    """Small pools and long generations: contention, holes, and (paged) preemption."""
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 24))
    block = int(rng.choice([4, 8, 16]))
    max_new = int(rng.integers(8, 64))
    prompts = rng.integers(0, 40, n)
    gens = rng.integers(1, max_new + 1, n)
    need = max(int(prompts.max()) + max_new, -(-int((prompts + gens).max()) // block) * block)
    total = -(-int(need * rng.uniform(1.0, 3.0)) // block) * block
    for policy in (ar.CONTIGUOUS, ar.PAGED):
        _same(policy, prompts, gens, max_new, total, block)


def test_hand_scenarios_match():
    _same(ar.PAGED, [15, 15], [20, 5], 20, 48)          # preemption every second step
    _same(ar.PAGED, [15, 15, 16], [20, 5, 1], 20, 48)   # preempted request back in front
    _same(ar.CONTIGUOUS, [16, 16, 16, 16, 52], [2, 4, 6, 3, 1], 20, 128)  # first fit, merge
    _same(ar.CONTIGUOUS, [16, 100, 16], [10, 1, 1], 20, 128)              # no overtaking
    got = _same(ar.PAGED, [15, 15], [20, 5], 20, 48)
    assert got["preemptions"] == 9


def test_preemption_happens_in_random_cases():
    """At least some of the random pools must exercise preemption (else the comparison
    above would not cover it)."""
    seen = 0
    for seed in range(12):
        rng = np.random.default_rng(100 + seed)
        n = int(rng.integers(1, 24))
        block = int(rng.choice([4, 8, 16]))
        max_new = int(rng.integers(8, 64))
        prompts = rng.integers(0, 40, n)
        gens = rng.integers(1, max_new + 1, n)
        need = max(int(prompts.max()) + max_new, -(-int((prompts + gens).max()) // block) * block)
        total = -(-int(need * rng.uniform(1.0, 3.0)) // block) * block
        seen += ar.replay(ar.PAGED, prompts, gens, max_new, total, block).preemptions > 0
    assert seen >= 3


def test_errors():
    from paged_kv_cache_200_amd import _lib
    rp = _native()
    with pytest.raises(_lib.PkvError):          # cannot fit an empty pool
        rp.replay_allocator(rp.PAGED, [15], [20], 20, 32)
    with pytest.raises(_lib.PkvError):
        rp.replay_allocator(rp.CONTIGUOUS, [100], [1], 192, 256)
    with pytest.raises(_lib.PkvError):          # gen above max_new
        rp.replay_allocator(rp.PAGED, [1], [30], 20, 256)
    with pytest.raises(_lib.PkvError):          # unknown policy
        rp.replay_allocator(7, [1], [1], 20, 256)
    with pytest.raises(_lib.PkvError):          # pool not a whole number of blocks
        rp.replay_allocator(rp.PAGED, [1], [1], 20, 250)
    assert rp.replay_allocator(rp.PAGED, [], [], 20, 256)["steps"] == 0
