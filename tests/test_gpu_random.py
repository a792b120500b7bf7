"""Randomised GPU parity against the oracle for the shared-prefix decode and the paged
prefill: random fork structures, sharing hints (true, short, over-stated, zero, members
copied away), partition sizes, chunk/context mixes and head shapes, several seeds each."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_util import assert_no_device_error, assert_parity, dev, oracle_decode, say
from libpkv_util import ensure_built
from oracle import paged_prefill as pp
from workloads import bf16_bits, build_case, fork_case

pytestmark = pytest.mark.gpu

SHAPES = [(32, 8, 128), (14, 2, 64), (8, 8, 64), (16, 2, 128), (6, 3, 64)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ensure_built()


def _copy_away(case, s, nblocks, rng):
    """Give sequence s fresh copies of its first nblocks blocks (same bits, new ids)."""
    used = set()
    for r, n in enumerate(case.context_lens.tolist()):
        used.update(case.block_tables[r, :-(-n // 16)].tolist())
    free = [b for b in range(case.num_blocks) if b not in used and b != case.poison_block]
    rng.shuffle(free)
    for j in range(min(nblocks, len(free))):
        src, dst = int(case.block_tables[s, j]), free.pop()
        case.k_pool[:, dst] = case.k_pool[:, src]
        case.v_pool[:, dst] = case.v_pool[:, src]
        case.block_tables[s, j] = dst


@pytest.mark.parametrize("seed", range(8))
def test_shared_prefix_random(seed):
    from paged_kv_cache_200_amd import ops
    rng = np.random.default_rng(1000 + seed)
    hq, hkv, d = SHAPES[seed % len(SHAPES)]
    parents = int(rng.integers(1, 6))
    forks = [int(rng.integers(1, 7)) for _ in range(parents)]
    prefixes, privates = [], []
    for f in forks:
        aligned = rng.random() < 0.7
        pre = int(rng.integers(1, 40)) * 16 if aligned else int(rng.integers(1, 500))
        prefixes.append(pre)
        privates.append([int(rng.integers(0, 300)) if aligned else 0 for _ in range(f)])
    case = fork_case("rand", prefixes, forks, privates, hq, hkv, d, "bf16", seed=seed,
                     pool_factor=3.0)
    starts = np.concatenate([[0], np.cumsum(forks)]).astype(np.int32)
    hint_kind = seed % 4
    shared = []
    for pre in prefixes:
        full = pre // 16
        shared.append({0: full, 1: max(0, full - 1), 2: full + 3, 3: 0}[hint_kind])
    if hint_kind == 2 and case.batch > 1:
        _copy_away(case, int(rng.integers(0, case.batch)), 4, rng)   # a stale hint too
    P = int(rng.choice([0, 16, 64, 512]))
    say(f"shared random seed {seed}: groups {forks} prefixes {prefixes} hint {hint_kind} P {P}")
    o, l = ops.paged_decode_shared_prefix(
        dev(case.q[0]), dev(case.k_pool[0]), dev(case.v_pool[0]), dev(case.block_tables),
        dev(case.context_lens), dev(starts), dev(np.asarray(shared, np.int32)),
        int(max(shared)), int(case.context_lens.max()), scale=float(case.scale),
        partition_size=P)
    torch.cuda.synchronize()
    assert_parity((o.cpu().numpy(), l.cpu().numpy()), oracle_decode(case), "bf16",
                  f"shared random {seed}")
    assert_no_device_error()


@pytest.mark.parametrize("seed", range(8))
def test_prefill_random(seed):
    from paged_kv_cache_200_amd import ops
    rng = np.random.default_rng(2000 + seed)
    hq, hkv, d = SHAPES[seed % len(SHAPES)]
    kv_dtype = "f32" if seed % 4 == 3 else "bf16"
    B = int(rng.integers(1, 7))
    lens = rng.integers(1, 700, B)
    chunks = np.array([int(rng.integers(0, n + 1)) if rng.random() < 0.8 else int(n)
                       for n in lens])
    case = build_case("rand", lens.astype(np.int32), hq, hkv, d, kv_dtype, seed)
    T = int(chunks.sum())
    x = rng.standard_normal((T, hq, d)).astype(np.float32)
    q = x if kv_dtype == "f32" else bf16_bits(x)
    cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    say(f"prefill random seed {seed}: {kv_dtype} {hq}/{hkv}x{d} lens {lens.tolist()} "
        f"chunks {chunks.tolist()}")
    want = pp.paged_prefill(q, case.k_pool[0], case.v_pool[0], case.block_tables, cu,
                            case.context_lens, case.scale, kv_dtype)
    if T == 0:
        return
    o, l = ops.paged_prefill(dev(q), dev(case.k_pool[0]), dev(case.v_pool[0]),
                             dev(case.block_tables), dev(cu), dev(case.context_lens),
                             int(chunks.max()), scale=float(case.scale))
    torch.cuda.synchronize()
    assert_parity((o.cpu().numpy(), l.cpu().numpy()), want, kv_dtype, f"prefill random {seed}")
    assert_no_device_error()
