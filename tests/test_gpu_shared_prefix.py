"""GPU parity of the shared-prefix decode (copy-on-write fork groups) against the
oracle's plain decode, including wrong sharing hints and malformed groups."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_util import DeviceCase, assert_no_device_error, assert_parity, dev, oracle_decode, say
from libpkv_util import ensure_built
from workloads import build_case, config_case, fork_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ensure_built()


def _shared_decode(dc, starts, shared, P, max_shared=None):
    from paged_kv_cache_200_amd import ops
    case = dc.case
    starts = np.asarray(starts, np.int32)
    shared = np.asarray(shared, np.int32)
    ms = int(shared.max()) if max_shared is None else max_shared
    o, l = ops.paged_decode_shared_prefix(dc.q, dc.k, dc.v, dc.tables, dc.ctx, dev(starts),
                                          dev(shared), ms, dc.max_ctx, scale=float(case.scale),
                                          partition_size=P)
    torch.cuda.synchronize()
    return o.cpu().numpy().astype(np.float64), l.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("P", [0, 512, 2048])
def test_prefix_fork_workload(P):
    say(f"prefix_fork shared-prefix decode P={P}")
    case = config_case("prefix_fork", 0)
    dc = DeviceCase(case)
    starts = np.arange(0, case.batch + 1, 4)
    shared = np.full(16, 2048 // 16)
    assert_parity(_shared_decode(dc, starts, shared, P), oracle_decode(case), "bf16",
                  f"shared prefix P{P}")
    assert_no_device_error()


@pytest.mark.parametrize("P", [0, 32, 256])
@pytest.mark.parametrize("kv_dtype,hq,hkv,d", [("bf16", 32, 8, 128), ("f32", 12, 12, 64),
                                               ("bf16", 14, 2, 64)])
@pytest.mark.parametrize("round_up", [False, True])
def test_mixed_groups(P, kv_dtype, hq, hkv, d, round_up):
    """Groups of 1, 2, 5 and 8 members (more members than a workgroup's waves), aligned
    prefixes with members that have no private token, an unaligned prefix whose shared
    hint is rounded down or up to whole blocks."""
    say(f"mixed groups P={P} {kv_dtype} {hq}/{hkv}x{d} round_up={round_up}")
    prefixes = [32, 20, 48, 400]
    forks = [1, 2, 5, 8]
    privates = [[37], [0, 0], [0, 16, 3, 70, 1], [5, 0, 290, 17, 64, 33, 2, 150]]
    case = fork_case("mixed", prefixes, forks, privates, hq, hkv, d, kv_dtype, seed=P + d)
    starts = np.concatenate([[0], np.cumsum(forks)])
    shared = [(-(-n // 16) if round_up else n // 16) for n in prefixes]
    dc = DeviceCase(case)
    assert_parity(_shared_decode(dc, starts, shared, P), oracle_decode(case), kv_dtype,
                  f"mixed groups P{P}")
    assert_no_device_error()


@pytest.mark.parametrize("P", [0, 8192])
@pytest.mark.parametrize("kv_dtype", ["bf16", "f32"])
def test_long_shared_prefix_across_id_windows(P, kv_dtype):
    """A shared prefix of more than 4096 tokens: the matrix-core tile reads 64 block ids
    per wave at a time (256 per tile), so its shared range crosses id windows."""
    say(f"long shared prefix P={P} {kv_dtype}")
    prefixes = [5008, 4112]
    forks = [3, 2]
    privates = [[7, 0, 130], [33, 1]]
    case = fork_case("longshared", prefixes, forks, privates, 16, 4, 128, kv_dtype, seed=P + 5)
    starts = np.concatenate([[0], np.cumsum(forks)])
    shared = [n // 16 for n in prefixes]
    dc = DeviceCase(case)
    assert_parity(_shared_decode(dc, starts, shared, P), oracle_decode(case), kv_dtype,
                  f"long shared prefix P{P}")
    assert_no_device_error()


def test_wrong_hint_and_clamp_still_exact():
    """A sharing hint that is not true (members hold different blocks), a bound below the
    hint, and members shorter than the declared prefix: results stay the plain decode."""
    case = build_case("indep", [100, 40, 300, 17, 256, 5], 8, 2, 128, "bf16", seed=12)
    dc = DeviceCase(case)
    want = oracle_decode(case)
    for starts, shared, ms in (([0, 3, 6], [16, 2], None), ([0, 6], [4], 2),
                               ([0, 1, 2, 3, 4, 5, 6], [0, 0, 0, 0, 0, 0], 0)):
        assert_parity(_shared_decode(dc, starts, shared, 64, ms), want, "bf16",
                      f"hint {shared} bound {ms}")
    assert_no_device_error()


def test_malformed_groups_flag_an_error():
    from paged_kv_cache_200_amd import ops
    case = build_case("bad", [10, 20, 30, 40], 4, 4, 64, "f32", seed=2)
    dc = DeviceCase(case)
    for starts in ([0, 3, 2, 4], [1, 2, 4], [0, 2, 3]):
        _shared_decode(dc, starts, [1] * (len(starts) - 1), 32)
        flags = ops.device_error()
        assert flags & 32, (starts, flags)
    assert_no_device_error()


@pytest.mark.parametrize("P", [0, 64, 512])
def test_copied_member_with_stale_hint(P):
    """One member of a real fork group had its prefix blocks copied (same contents, new
    ids) while the hint still counts them as shared; a sibling is shorter than the prefix.
    Outputs must equal the plain decode."""
    say(f"copied member, stale hint, P={P}")
    case = fork_case("copied", [96, 160], [4, 3], [[0, 16, 40, 3], [7, 0, 33]], 32, 8, 128,
                     "bf16", seed=21, pool_factor=3.0)
    refs = {}
    for s, n in enumerate(case.context_lens.tolist()):
        for j in range(-(-n // 16)):
            refs.setdefault(int(case.block_tables[s, j]), []).append(s)
    free = [b for b in range(case.num_blocks) if b not in refs and b != case.poison_block]
    victim = 2  # third member of the first group
    for j in range(96 // 16):
        src, dst = int(case.block_tables[victim, j]), free.pop()
        case.k_pool[:, dst] = case.k_pool[:, src]
        case.v_pool[:, dst] = case.v_pool[:, src]
        case.block_tables[victim, j] = dst
    case.context_lens[1] = 40  # shorter than the 96-token prefix: stops inside it
    starts = [0, 4, 7]
    dc = DeviceCase(case)
    assert_parity(_shared_decode(dc, starts, [6, 10], P), oracle_decode(case), "bf16",
                  f"copied member P{P}")
    assert_no_device_error()


@pytest.mark.parametrize("P", [0, 256])
def test_append_and_shared_decode_in_one_call(P):
    """append_paged_decode_shared_prefix == kv_append, then paged_decode_shared_prefix
    (bit for bit), and the appended cache equals the oracle's append."""
    from oracle import paged_attention as pa
    from paged_kv_cache_200_amd import ops
    say(f"append + shared decode in one call, P={P}")
    prefixes, forks = [64, 128], [3, 2]
    privates = [[5, 16, 30], [1, 47]]
    case = fork_case("append", prefixes, forks, privates, 32, 8, 128, "bf16", seed=4)
    B, hkv, d = case.batch, case.num_kv_heads, case.head_dim
    rng = np.random.default_rng(9)
    # one new token per member, at its last position (inside its private blocks)
    start = (case.context_lens - 1).astype(np.int32)
    cu = np.arange(B + 1, dtype=np.int32)
    kn = (rng.standard_normal((B, hkv, d), dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    vn = (rng.standard_normal((B, hkv, d), dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    starts = np.array([0, 3, 5], np.int32)
    shared = np.array([4, 8], np.int32)
    results = []
    for fused in (True, False):
        dc = DeviceCase(case)
        args = (dev(kn), dev(vn), dc.tables, dev(start), dev(cu))
        if fused:
            o, l = ops.append_paged_decode_shared_prefix(
                dc.q, dc.k, dc.v, *args, dc.ctx, dev(starts), dev(shared), 8, dc.max_ctx,
                scale=float(case.scale), partition_size=P)
        else:
            ops.kv_append(dc.k, dc.v, *args)
            o, l = ops.paged_decode_shared_prefix(dc.q, dc.k, dc.v, dc.tables, dc.ctx,
                                                  dev(starts), dev(shared), 8, dc.max_ctx,
                                                  scale=float(case.scale), partition_size=P)
        torch.cuda.synchronize()
        results.append((o.cpu().numpy(), l.cpu().numpy(), dc.k.cpu().numpy(), dc.v.cpu().numpy()))
    for a, b in zip(results[0], results[1]):
        assert a.tobytes() == b.tobytes()
    k2, v2 = pa.kv_append(case.k_pool[0], case.v_pool[0], kn, vn, case.block_tables, start, cu)
    assert results[0][2].view(np.uint16).tobytes() == k2.tobytes()
    assert results[0][3].view(np.uint16).tobytes() == v2.tobytes()
    want = pa.paged_decode(case.q[0], k2, v2, case.block_tables, case.context_lens, case.scale,
                           "bf16")
    assert_parity((results[0][0].astype(np.float64), results[0][1].astype(np.float64)), want,
                  "bf16", f"append+shared P{P}")
    assert_no_device_error()
