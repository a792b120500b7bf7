"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Indexing (append, block copy, the one-hot gather probe,
batched-vs-alone, forks) must be bit-exact; attention values within 2e-3
max-abs for fp32 caches and 1e-2 for bf16 caches (fp32 accumulation)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.paged_attention as pa
from gpu_util import (TOL, DeviceCase, assert_no_device_error, assert_parity, dev, host_bits,
                      oracle_decode, run_decode, say)
from libpkv_util import ensure_built
from workloads import bf16_bits, build_case, config_case, fork_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ensure_built()
    import paged_kv_cache_200_amd  # noqa: F401


def _ops():
    from paged_kv_cache_200_amd import ops
    return ops


# --------------------------------------------------------------------------------------
# KV append and block copy: bit-exact
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("kv_dtype,hkv,d", [("f32", 12, 64), ("bf16", 2, 64), ("bf16", 8, 128),
                                            ("f32", 4, 128)])
def test_append_bitexact(kv_dtype, hkv, d):
    say(f"append {kv_dtype} hkv={hkv} d={d}")
    rng = np.random.default_rng(hkv * 1000 + d)
    case = build_case("append", [40, 100, 1, 77, 200], hkv, hkv, d, kv_dtype, seed=d + hkv)
    B = case.batch
    # a prefill-like write of several tokens per sequence at explicit starts, some
    # crossing block boundaries, one empty, then a one-token decode write
    for starts, counts in (([0, 13, 0, 60, 150], [16, 40, 1, 0, 33]),
                           (list(case.context_lens - 1), [1] * B)):
        starts = np.array(starts, np.int32)
        cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        x = rng.standard_normal((int(cu[-1]), hkv, d)).astype(np.float32)
        y = rng.standard_normal((int(cu[-1]), hkv, d)).astype(np.float32)
        if kv_dtype == "bf16":
            x, y = bf16_bits(x), bf16_bits(y)
        kd, vd = dev(case.k_pool[0]), dev(case.v_pool[0])
        _ops().kv_append(kd, vd, dev(x), dev(y), dev(case.block_tables), dev(starts), dev(cu))
        want_k, want_v = pa.kv_append(case.k_pool[0], case.v_pool[0], x, y, case.block_tables,
                                      starts, cu)
        assert host_bits(kd, kv_dtype).tobytes() == want_k.tobytes()
        assert host_bits(vd, kv_dtype).tobytes() == want_v.tobytes()
    assert_no_device_error()


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16"])
def test_copy_blocks_bitexact(kv_dtype):
    case = build_case("copy", [64, 64, 64], 4, 4, 128, kv_dtype, seed=3, layers=3)
    k = dev(case.k_pool)
    v = dev(case.v_pool)
    src, dst = [0, 5, 2], [7, 1, 9]
    _ops().copy_blocks(k, v, dev(np.array(src, np.int32)), dev(np.array(dst, np.int32)))
    for layer in range(3):
        wk, wv = pa.copy_blocks(case.k_pool[layer], case.v_pool[layer], src, dst)
        assert host_bits(k[layer], kv_dtype).tobytes() == wk.tobytes()
        assert host_bits(v[layer], kv_dtype).tobytes() == wv.tobytes()
    # one layer at a time
    k1 = dev(case.k_pool[0])
    v1 = dev(case.v_pool[0])
    _ops().copy_blocks(k1, v1, dev(np.array(src, np.int32)), dev(np.array(dst, np.int32)))
    wk, wv = pa.copy_blocks(case.k_pool[0], case.v_pool[0], src, dst)
    assert host_bits(k1, kv_dtype).tobytes() == wk.tobytes()
    assert_no_device_error()


# --------------------------------------------------------------------------------------
# Decode parity on the workload configs
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("P", [0, 16, 64, 512])
def test_decode_tiny(seed, P):
    say(f"tiny seed={seed} P={P}")
    case = config_case("tiny", seed)
    assert_parity(run_decode(DeviceCase(case), P), oracle_decode(case), "f32", f"tiny s{seed}")
    assert_no_device_error()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_qwen_gqa(seed):
    layers = 24 if seed == 0 else 3
    say(f"qwen_gqa seed={seed} layers={layers}")
    case = config_case("qwen_gqa", seed, layers=layers)
    for layer in range(layers):
        for P in ((0, 256) if layer % 6 == 0 else (256,)):
            assert_parity(run_decode(DeviceCase(case, layer), P), oracle_decode(case, layer),
                          "bf16", f"qwen s{seed} L{layer} P{P}")
    assert_no_device_error()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_high_concurrency(seed):
    say(f"high_concurrency seed={seed}")
    case = config_case("high_concurrency", seed)
    want = oracle_decode(case)
    dc = DeviceCase(case)
    for P in (512,) if seed else (512, 256, 0):
        assert_parity(run_decode(dc, P), want, "bf16", f"C4 s{seed} P{P}")
    assert_no_device_error()


def test_decode_prefix_fork():
    say("prefix_fork")
    case = config_case("prefix_fork", 0)
    assert_parity(run_decode(DeviceCase(case), 512), oracle_decode(case), "bf16", "C5a")
    assert_no_device_error()


def test_decode_long_context():
    say("long_context")
    case = config_case("long_context", 0)
    assert_parity(run_decode(DeviceCase(case), 512), oracle_decode(case), "bf16", "C5b P512")
    assert_no_device_error()


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("P", [16, 512])
def test_partials_and_combine(kv_dtype, P):
    case = build_case("parts", [0, 1, 15, 16, 17, 511, 512, 513, 1500], 8, 2, 128, kv_dtype, 5)
    dc = DeviceCase(case)
    ops = _ops()
    po, pl = ops.paged_decode_partials(dc.q, dc.k, dc.v, dc.tables, dc.ctx, dc.max_ctx, P,
                                       scale=float(case.scale), max_partitions=None)
    wpo, wpl = pa.decode_partitions(case.q[0], case.k_pool[0], case.v_pool[0],
                                    case.block_tables, case.context_lens, case.scale, kv_dtype, P)
    # entries past a sequence's last partition are not written: compare the live ones
    live = np.zeros(wpl.shape, bool)
    for s, n in enumerate(case.context_lens.tolist()):
        live[s, :, :max(1, -(-n // P))] = True
    gpo, gpl = po.cpu().numpy(), pl.cpu().numpy()
    assert_parity((gpo[live], gpl[live]), (wpo[live], wpl[live]), kv_dtype, f"partials P{P}")
    o, l = ops.lse_combine(po, pl, dc.ctx, P)
    assert_parity((o.cpu().numpy(), l.cpu().numpy()), pa.combine_partitions(wpo, wpl), kv_dtype,
                  f"combine P{P}")
    assert_parity((o.cpu().numpy(), l.cpu().numpy()), oracle_decode(case), kv_dtype, "vs unsplit")
    assert_no_device_error()


# --------------------------------------------------------------------------------------
# Edge cases
# --------------------------------------------------------------------------------------

BOUNDARY_LENS = [1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 255, 256, 257, 511, 512, 513, 1023,
                 1024, 1025, 2047]


@pytest.mark.parametrize("kv_dtype,hq,hkv,d", [("bf16", 32, 8, 128), ("f32", 12, 12, 64),
                                               ("bf16", 14, 2, 64), ("bf16", 8, 8, 128),
                                               ("f32", 16, 2, 128), ("bf16", 5, 1, 64)])
@pytest.mark.parametrize("P", [0, 64, 512])
def test_block_and_partition_boundaries(kv_dtype, hq, hkv, d, P):
    case = build_case("bounds", BOUNDARY_LENS, hq, hkv, d, kv_dtype, seed=hq + d + P)
    assert_parity(run_decode(DeviceCase(case), P), oracle_decode(case), kv_dtype,
                  f"bounds {kv_dtype} G{hq // hkv} D{d} P{P}")
    assert_no_device_error()


# A wave reads its block ids 64 at a time; with four waves a unit longer than 4096 tokens
# (P = 0, or a large partition) crosses id windows, with odd and even block counts left
# for the last window and a partial last block.
WINDOW_LENS = [9000, 8193, 4112, 4097, 4096, 300]


@pytest.mark.parametrize("kv_dtype,hq,hkv,d", [("bf16", 32, 8, 128), ("f32", 8, 2, 64),
                                               ("bf16", 14, 2, 64)])
@pytest.mark.parametrize("P", [0, 8192])
def test_units_across_id_windows(kv_dtype, hq, hkv, d, P):
    case = build_case("windows", WINDOW_LENS, hq, hkv, d, kv_dtype, seed=hq + d + P + 7)
    assert_parity(run_decode(DeviceCase(case), P), oracle_decode(case), kv_dtype,
                  f"id windows {kv_dtype} G{hq // hkv} D{d} P{P}")
    assert_no_device_error()


@pytest.mark.parametrize("P", [0, 32])
def test_empty_contexts(P):
    case = build_case("empty", [0, 5, 0, 40, 0], 8, 2, 64, "bf16", seed=1)
    o, l = run_decode(DeviceCase(case), P)
    assert np.all(o[[0, 2, 4]] == 0) and np.all(l[[0, 2, 4]] == -np.inf)
    assert_parity((o, l), oracle_decode(case), "bf16", f"empty P{P}")
    allzero = build_case("allempty", [0, 0], 4, 4, 64, "f32", seed=2)
    o, l = run_decode(DeviceCase(allzero), P)
    assert np.all(o == 0) and np.all(l == -np.inf)
    assert_no_device_error()


def test_max_context_len_above_true_max():
    case = build_case("slack", [100, 700, 33], 8, 2, 128, "bf16", seed=4, table_width=200)
    want = oracle_decode(case)
    dc = DeviceCase(case)
    for max_ctx in (700, 701, 1024, 3200):
        assert_parity(run_decode(dc, 64, max_ctx=max_ctx), want, "bf16", f"max_ctx {max_ctx}")
    assert_no_device_error()


@pytest.mark.parametrize("q_scale", [8.0, 30.0])
@pytest.mark.parametrize("kv_dtype", ["f32", "bf16"])
def test_softmax_stability(q_scale, kv_dtype):
    case = build_case("stable", [3, 90, 600, 1300], 16, 4, 128 if kv_dtype == "bf16" else 64,
                      kv_dtype, seed=9, q_scale=q_scale)
    want = oracle_decode(case)
    dc = DeviceCase(case)
    for P in (0, 128):
        assert_parity(run_decode(dc, P), want, kv_dtype, f"q x{q_scale} P{P}")
    assert_no_device_error()


@pytest.mark.parametrize("kv_dtype,d", [("bf16", 128), ("f32", 64), ("bf16", 64)])
@pytest.mark.parametrize("P", [0, 64])
def test_one_hot_gather_probe_bitwise(kv_dtype, d, P):
    """One token per sequence scores >= 100 above all others: out must be that
    token's V row exactly, which makes the gather's indexing bit-checkable."""
    lens = [1, 17, 130, 700]
    case = build_case("probe", lens, 4, 2, d, kv_dtype, seed=d + P)
    rng = np.random.default_rng(7)
    kp = case.k_pool[0].copy()
    q = np.zeros_like(case.q[0])
    one = np.float32(1.0) if kv_dtype == "f32" else bf16_bits(np.float32(1.0))
    big = np.float32(160.0) if kv_dtype == "f32" else bf16_bits(np.float32(160.0))
    small = np.float32(0.0) if kv_dtype == "f32" else bf16_bits(np.float32(0.0))
    q[:, :, 0] = one
    hot = []
    for s, n in enumerate(lens):
        t = int(rng.integers(n))
        hot.append(t)
        for tt in range(n):
            blk, slot = case.block_tables[s, tt // 16], tt % 16
            kp[blk, :, slot, 0] = big if tt == t else small
    case.k_pool = kp[None]
    case.q = q[None]
    case.scale = np.float32(1.0)
    o, l = run_decode(DeviceCase(case), P)
    vals = pa.widen(case.v_pool[0], kv_dtype)
    G = 2
    for s, t in enumerate(hot):
        blk, slot = case.block_tables[s, t // 16], t % 16
        for h in range(4):
            row = vals[blk, h // G, slot].astype(np.float32)
            assert o[s, h].astype(np.float32).tobytes() == row.tobytes(), (s, h)
    assert_no_device_error()


@pytest.mark.parametrize("P", [0, 64, 512])
def test_batched_equals_alone_bitwise(P):
    """A sequence decoded in a batch or alone gives bit-identical out and lse
    (no attention leaks across sequence boundaries)."""
    case = config_case("high_concurrency", 1, max_batch=24)
    dc = DeviceCase(case)
    ob, lb = run_decode(dc, P)
    ops = _ops()
    for s in range(case.batch):
        o, l = ops.paged_decode(dc.q[s:s + 1], dc.k, dc.v, dc.tables[s:s + 1].contiguous(),
                                dc.ctx[s:s + 1].contiguous(), int(case.context_lens[s]),
                                scale=float(case.scale), partition_size=P)
        assert o.cpu().numpy().tobytes() == ob[s:s + 1].astype(np.float32).tobytes(), s
        assert l.cpu().numpy().tobytes() == lb[s:s + 1].astype(np.float32).tobytes(), s
    assert_no_device_error()


def test_forks_bitwise_identical():
    case = fork_case("forks", [2048, 40, 500], 4, [[0] * 4] * 3, 32, 8, 128, "bf16", seed=3)
    q = case.q[0].copy()
    for s in range(case.batch):
        q[s] = q[case.fork_parent[s] * 4]
    case.q = q[None]
    for P in (0, 512):
        o, l = run_decode(DeviceCase(case), P)
        for s in range(case.batch):
            f0 = case.fork_parent[s] * 4
            assert o[s].tobytes() == o[f0].tobytes() and l[s].tobytes() == l[f0].tobytes()
        assert_parity((o, l), oracle_decode(case), "bf16", f"forks P{P}")
    assert_no_device_error()


@pytest.mark.parametrize("fill", ["inf", "huge"])
def test_stale_slots_never_leak(fill):
    """Unowned slots holding inf or huge values instead of NaN change nothing."""
    case = build_case("stale", [5, 16, 33, 250], 8, 2, 64, "f32", seed=11)
    ref = run_decode(DeviceCase(case), 64)
    kp, vp = case.k_pool.copy(), case.v_pool.copy()
    val = np.float32(np.inf) if fill == "inf" else np.float32(3e38)
    nan_k = np.isnan(kp)
    kp[nan_k] = val
    vp[np.isnan(vp)] = -val
    case.k_pool, case.v_pool = kp, vp
    got = run_decode(DeviceCase(case), 64)
    assert got[0].tobytes() == ref[0].tobytes() and got[1].tobytes() == ref[1].tobytes()
    assert_parity(got, oracle_decode(case), "f32", f"stale {fill}")
    assert_no_device_error()


# --------------------------------------------------------------------------------------
# Work plan: order only, never results
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("P", [0, 256])
def test_plan_reused_across_layers(P):
    """One plan per step serves every layer: planned calls equal the all-in-one call
    bit for bit, and the oracle within tolerance."""
    case = config_case("qwen_gqa", 1, layers=3)
    ops = _ops()
    dcs = [DeviceCase(case, layer) for layer in range(3)]
    ws = ops.decode_plan(dcs[0].ctx, dcs[0].tables, case.num_q_heads, case.head_dim,
                         dcs[0].max_ctx, P)
    for layer, dc in enumerate(dcs):
        o1, l1 = ops.paged_decode_planned(dc.q, dc.k, dc.v, dc.tables, dc.ctx, dc.max_ctx, ws,
                                          scale=float(case.scale), partition_size=P)
        o2, l2 = ops.paged_decode(dc.q, dc.k, dc.v, dc.tables, dc.ctx, dc.max_ctx,
                                  scale=float(case.scale), partition_size=P)
        torch.cuda.synchronize()
        assert o1.cpu().numpy().tobytes() == o2.cpu().numpy().tobytes()
        assert l1.cpu().numpy().tobytes() == l2.cpu().numpy().tobytes()
        assert_parity((o1.cpu().numpy(), l1.cpu().numpy()), oracle_decode(case, layer), "bf16",
                      f"planned L{layer} P{P}")
    assert_no_device_error()


def test_partials_with_and_without_plan_identical():
    case = config_case("high_concurrency", 2, max_batch=40)
    dc = DeviceCase(case)
    ops = _ops()
    P = 128
    a = ops.paged_decode_partials(dc.q, dc.k, dc.v, dc.tables, dc.ctx, dc.max_ctx, P,
                                  scale=float(case.scale))
    ws = ops.decode_plan(dc.ctx, dc.tables, case.num_q_heads, case.head_dim, dc.max_ctx, P)
    b = ops.paged_decode_partials(dc.q, dc.k, dc.v, dc.tables, dc.ctx, dc.max_ctx, P,
                                  scale=float(case.scale), plan_workspace=ws)
    torch.cuda.synchronize()
    live = np.zeros(a[1].shape, bool)
    for s, n in enumerate(case.context_lens.tolist()):
        live[s, :, :max(1, -(-n // P))] = True
    assert a[0].cpu().numpy()[live].tobytes() == b[0].cpu().numpy()[live].tobytes()
    assert a[1].cpu().numpy()[live].tobytes() == b[1].cpu().numpy()[live].tobytes()
    assert_no_device_error()


@pytest.mark.parametrize("P", [0, 64, 1024])
def test_plan_lists_every_unit_once_in_order(P):
    """Plan layout inside the workspace: int32 count at byte 0; from byte 256 int4
    entries (sequence, first token, end token, slot | 1<<30 when the unit is the
    sequence's only one and writes the output itself); then one int32 per sequence,
    the number of slots the combine merges (0 for a direct sequence)."""
    lens = [0, 1, 15, 16, 17, 64, 65, 130, 1024, 1025, 3000, 5, 700, 64]
    case = build_case("plan", lens, 8, 2, 64, "bf16", seed=3)
    dc = DeviceCase(case)
    ws = _ops().decode_plan(dc.ctx, dc.tables, 8, 64, dc.max_ctx, P)
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()
    count = int(raw[:4].view(np.int32)[0])
    split = P > 0 and dc.max_ctx > P
    max_slots = -(-dc.max_ctx // P) if split else 1
    ent = raw[256:256 + 16 * count].view(np.int32).reshape(-1, 4).tolist()
    off = 256 + -(-len(lens) * max_slots * 16 // 256) * 256
    nslots = raw[off:off + 4 * len(lens)].view(np.int32).tolist()
    direct = 1 << 30
    per_seq = {}
    for s_, t0, t1, w in ent:
        per_seq.setdefault(s_, []).append((t0, t1, w))
    assert sorted(per_seq) == list(range(len(lens)))
    for s_, n in enumerate(lens):
        units = sorted(per_seq[s_])
        want = [(p * P, min((p + 1) * P, n)) for p in range(max(1, -(-n // P)))] \
            if split else [(0, n)]
        assert [(t0, t1) for t0, t1, _ in units] == want, s_
        if len(want) == 1:
            assert units[0][2] == direct and nslots[s_] == 0, s_
        else:
            assert [w for _, _, w in units] == list(range(len(want))), s_
            assert nslots[s_] == len(want), s_
    assert count == sum(len(v) for v in per_seq.values())
    # order: every full partition, then the last unit of every split sequence (merged
    # early), then the other units longest first
    rank = []
    for s_, t0, t1, _ in ent:
        if split and t1 - t0 == P:
            rank.append(0)
        elif len(per_seq[s_]) > 1:
            rank.append(1)
        else:
            rank.append(2)
    assert rank == sorted(rank), "full partitions, then split sequences' last units, first"
    rest = [-(-(t1 - t0) // 16) for (_, t0, t1, _), r in zip(ent, rank) if r == 2]
    assert rest == sorted(rest, reverse=True), "plan is not longest-first"
    assert_no_device_error()


# --------------------------------------------------------------------------------------
# The all-in-one call equals first pass + standalone combine, on every call
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("P", [64, 512, 2048])
def test_decode_equals_partials_plus_combine_bitwise(P):
    case = config_case("high_concurrency", 0)
    _check_decode_equals_partials_plus_combine(case, P)


@pytest.mark.parametrize("kv_dtype,hq,hkv,d,lens,P", [
    ("bf16", 14, 2, 64, [2297, 1, 512, 513, 1800, 40], 512),   # Qwen shape, up to 5 slots
    ("f32", 12, 12, 64, [192, 17, 100, 64], 32),                # 6 slots
    ("f32", 8, 2, 128, [700, 5, 256, 129], 128),                # 6 slots
    ("bf16", 32, 8, 128, [1024, 1023, 897, 9, 600], 128),       # 8 slots: the in-pass limit
    ("bf16", 32, 8, 128, [1152, 1151, 1025, 9, 600], 128),      # 9 slots: the combine launch
    ("bf16", 32, 8, 128, [2176, 2049, 600, 9], 128),            # 17: a last group of one
    ("bf16", 14, 2, 64, [2200, 1, 513, 40], 128),               # 18, matrix-core pass
    ("bf16", 32, 8, 128, [1024, 1000, 9], 16),                  # 64: the grouped combine
    ("f32", 12, 12, 64, [1040, 17, 300], 16),                   # 65: one wave per row
])
def test_decode_equals_partials_plus_combine_shapes(kv_dtype, hq, hkv, d, lens, P):
    """The merge of split sequences, inside the first pass up to 8 partitions and in the
    combine kernel past that (two steps from 9 to 64 partitions), equals the first pass's
    partials + the standalone combine, bit for bit, for every head shape it is compiled
    for here; and the oracle's result within tolerance."""
    case = build_case("merge", lens, hq, hkv, d, kv_dtype, seed=len(lens) + P)
    _check_decode_equals_partials_plus_combine(case, P)
    assert_parity(run_decode(DeviceCase(case), P), oracle_decode(case), kv_dtype, f"merge P{P}")


@pytest.mark.parametrize("d", [64, 128])
def test_combine_in_two_steps_on_either_kernel(d):
    """Rows of 9 to 64 partitions are merged in two steps (each group of 8 consecutive
    partitions, then the groups).  A call whose max_partitions is at most 64 runs them on
    one wave per group (lse_combine_grouped_kernel), a wider call on one wave per row:
    the same partials give the same bits either way, and the oracle's combine within
    float32 rounding.  Slots past a row's count hold NaN and must not be read; empty
    partitions (lse -inf) and an all-empty row are included."""
    say(f"combine in two steps, d {d}")
    ops = _ops()
    P, hq = 16, 3
    counts = [1, 5, 8, 9, 16, 17, 33, 63, 64, 40]
    B = len(counts)
    ctx = np.array([n * P - (n % 3) for n in counts], np.int32)
    rng = np.random.default_rng(d)
    po = rng.standard_normal((B, hq, 64, d)).astype(np.float32)
    pl = rng.uniform(-6.0, 6.0, (B, hq, 64)).astype(np.float32)
    pl[2, 0, 3] = -np.inf            # one empty partition in an 8-slot row
    pl[4, 1, :7] = -np.inf           # a whole first group empty
    pl[9, 2, :40] = -np.inf          # a row with nothing live
    for s, n in enumerate(counts):
        po[s, :, n:] = np.nan
        pl[s, :, n:] = np.nan
    wide_o = np.full((B, hq, 80, d), np.nan, np.float32)
    wide_l = np.full((B, hq, 80), np.nan, np.float32)
    wide_o[:, :, :64], wide_l[:, :, :64] = po, pl
    dctx = dev(ctx)
    o1, l1 = ops.lse_combine(dev(po), dev(pl), dctx, P)
    o2, l2 = ops.lse_combine(dev(wide_o), dev(wide_l), dctx, P)
    torch.cuda.synchronize()
    assert o1.cpu().numpy().tobytes() == o2.cpu().numpy().tobytes()
    assert l1.cpu().numpy().tobytes() == l2.cpu().numpy().tobytes()
    ref_l = pl.astype(np.float64)
    ref_o = np.nan_to_num(po.astype(np.float64))
    for s, n in enumerate(counts):
        ref_l[s, :, n:] = -np.inf
    want = pa.combine_partitions(ref_o, ref_l)
    got = (o1.cpu().numpy(), l1.cpu().numpy())
    assert np.array_equal(np.isneginf(got[1]), np.isneginf(want[1]))
    assert np.all(got[0][9, 2] == 0.0)
    assert np.max(np.abs(got[0] - want[0])) < 1e-5
    live = ~np.isneginf(want[1])
    assert np.max(np.abs(got[1][live] - want[1][live])) < 1e-5
    assert_no_device_error()


def _check_decode_equals_partials_plus_combine(case, P):
    dc = DeviceCase(case)
    ops = _ops()
    fo, fl = ops.paged_decode(dc.q, dc.k, dc.v, dc.tables, dc.ctx, dc.max_ctx,
                              scale=float(case.scale), partition_size=P)
    po, pl = ops.paged_decode_partials(dc.q, dc.k, dc.v, dc.tables, dc.ctx, dc.max_ctx, P,
                                       scale=float(case.scale))
    so, sl = ops.lse_combine(po, pl, dc.ctx, P)
    torch.cuda.synchronize()
    # sequences that fit one partition are written straight by the first pass in both
    assert fo.cpu().numpy().tobytes() == so.cpu().numpy().tobytes()
    assert fl.cpu().numpy().tobytes() == sl.cpu().numpy().tobytes()
    assert_no_device_error()


def test_decode_repeatable_with_reused_workspace():
    """Twenty calls on two alternating workspaces, with a plan reused in between:
    every result bit-identical (no stale partials or plan entries leak into a call)."""
    case = config_case("long_context", 0)
    dc = DeviceCase(case)
    ops = _ops()
    P = 512
    first = ops.paged_decode(dc.q, dc.k, dc.v, dc.tables, dc.ctx, dc.max_ctx,
                             scale=float(case.scale), partition_size=P)
    ref = (first[0].cpu().numpy().tobytes(), first[1].cpu().numpy().tobytes())
    need = ops.decode_workspace_bytes(case.batch, case.num_q_heads, case.head_dim, dc.max_ctx, P)
    wss = [torch.empty(need, dtype=torch.uint8, device="cuda") for _ in range(2)]
    ops.decode_plan(dc.ctx, dc.tables, case.num_q_heads, case.head_dim, dc.max_ctx, P,
                    workspace=wss[1])
    for i in range(20):
        if i % 2 == 0:
            o, l = ops.paged_decode(dc.q, dc.k, dc.v, dc.tables, dc.ctx, dc.max_ctx,
                                    scale=float(case.scale), partition_size=P, workspace=wss[0])
        else:
            o, l = ops.paged_decode_planned(dc.q, dc.k, dc.v, dc.tables, dc.ctx, dc.max_ctx,
                                            wss[1], scale=float(case.scale), partition_size=P)
        assert (o.cpu().numpy().tobytes(), l.cpu().numpy().tobytes()) == ref, f"call {i}"
    assert_no_device_error()


@pytest.mark.parametrize("P", [0, 512, 4096])
@pytest.mark.parametrize("kv_dtype", ["bf16", "f32"])
def test_append_paged_decode_equals_separate_calls(P, kv_dtype):
    """The one-call append + decode equals kv_append followed by paged_decode, bit for
    bit (outputs and pools), and the oracle within tolerance."""
    hkv, hq, d = (8, 32, 128) if kv_dtype == "bf16" else (12, 12, 64)
    case = build_case("step", [17, 1, 700, 4097, 64, 5000], hq, hkv, d, kv_dtype, seed=P + d)
    rng = np.random.default_rng(P)
    B = case.batch
    kn = rng.standard_normal((B, hkv, d)).astype(np.float32)
    vn = rng.standard_normal((B, hkv, d)).astype(np.float32)
    if kv_dtype == "bf16":
        kn, vn = bf16_bits(kn), bf16_bits(vn)
    start = (case.context_lens - 1).astype(np.int32)
    cu = np.arange(B + 1, dtype=np.int32)
    ops = _ops()
    a, b = DeviceCase(case), DeviceCase(case)
    o1, l1 = ops.append_paged_decode(a.q, a.k, a.v, dev(kn), dev(vn), a.tables, dev(start),
                                     dev(cu), a.ctx, a.max_ctx, scale=float(case.scale),
                                     partition_size=P)
    ops.kv_append(b.k, b.v, dev(kn), dev(vn), b.tables, dev(start), dev(cu))
    o2, l2 = ops.paged_decode(b.q, b.k, b.v, b.tables, b.ctx, b.max_ctx, scale=float(case.scale),
                              partition_size=P)
    torch.cuda.synchronize()
    assert o1.cpu().numpy().tobytes() == o2.cpu().numpy().tobytes()
    assert l1.cpu().numpy().tobytes() == l2.cpu().numpy().tobytes()
    assert a.k.cpu().numpy().tobytes() == b.k.cpu().numpy().tobytes()
    assert a.v.cpu().numpy().tobytes() == b.v.cpu().numpy().tobytes()
    kp, vp = pa.kv_append(case.k_pool[0], case.v_pool[0], kn, vn, case.block_tables, start, cu)
    want = pa.paged_decode(case.q[0], kp, vp, case.block_tables, case.context_lens, case.scale,
                           kv_dtype)
    assert_parity((o1.cpu().numpy(), l1.cpu().numpy()), want, kv_dtype, f"append+decode P{P}")
    assert_no_device_error()


@pytest.mark.parametrize("wl,P", [("long_context", 512), ("high_concurrency", 1024)])
def test_in_pass_merge_sees_this_calls_partials(wl, P):
    """Split sequences are merged inside the first pass by the last of their units to
    finish, reading the other units' partial results through device-scope loads.  A new
    query on every call, on one reused workspace and on one reused plan: each result must
    equal that query's first pass + standalone combine bit for bit, so a merge that read
    a previous call's partials (or a counter left unreset) fails."""
    case = config_case(wl, 1, max_batch=64)
    dc = DeviceCase(case)
    ops = _ops()
    rng = np.random.default_rng(P)
    need = ops.decode_workspace_bytes(case.batch, case.num_q_heads, case.head_dim, dc.max_ctx, P)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    plan_ws = ops.decode_plan(dc.ctx, dc.tables, case.num_q_heads, case.head_dim, dc.max_ctx, P)
    for i in range(6):
        qh = rng.standard_normal(case.q[0].shape).astype(np.float32)
        if case.kv_dtype == "bf16":
            qh = bf16_bits(qh)
        q = dev(qh)
        say(f"  {wl} P{P} call {i}")
        if i % 2 == 0:
            o, l = ops.paged_decode(q, dc.k, dc.v, dc.tables, dc.ctx, dc.max_ctx,
                                    scale=float(case.scale), partition_size=P, workspace=ws)
        else:
            o, l = ops.paged_decode_planned(q, dc.k, dc.v, dc.tables, dc.ctx, dc.max_ctx,
                                            plan_ws, scale=float(case.scale), partition_size=P)
        po, pl = ops.paged_decode_partials(q, dc.k, dc.v, dc.tables, dc.ctx, dc.max_ctx, P,
                                           scale=float(case.scale))
        so, sl = ops.lse_combine(po, pl, dc.ctx, P)
        torch.cuda.synchronize()
        assert o.cpu().numpy().tobytes() == so.cpu().numpy().tobytes(), f"call {i}"
        assert l.cpu().numpy().tobytes() == sl.cpu().numpy().tobytes(), f"call {i}"
        if i == 5:
            assert_parity((o.cpu().numpy(), l.cpu().numpy()), oracle_decode(case, q=qh),
                          case.kv_dtype, f"{wl} P{P}")
    assert_no_device_error()


@pytest.mark.parametrize("P", [0, 512, 4096])
@pytest.mark.parametrize("kv_dtype", ["bf16", "f32"])
def test_append_in_pass_equals_separate_calls(P, kv_dtype):
    """pkv_append_paged_decode_planned (the append written by the first pass itself) equals
    kv_append followed by paged_decode_planned, bit for bit (outputs and pools), for new
    tokens at the first and last slot of a block, at a partition's first token, in the
    middle of the attended range, past it, several per sequence and none; and the oracle
    within tolerance."""
    hkv, hq, d = (8, 32, 128) if kv_dtype == "bf16" else (12, 12, 64)
    lens = [1, 16, 17, 4097, 700, 512, 5000, 33, 64, 0, 60]
    case = build_case("step_in_pass", lens, hq, hkv, d, kv_dtype, seed=P + d + 1)
    B = case.batch
    # (start, count) per sequence: the last token, a whole last block, a partition's first
    # token, two tokens in the middle, none, one past the attended range, one into an empty
    # context, twenty across a block boundary
    spec = [(0, 1), (15, 1), (16, 1), (4096, 1), (698, 2), (0, 0), (4990, 3), (33, 1),
            (63, 1), (0, 1), (40, 20)]
    start = np.array([p for p, _ in spec], np.int32)
    counts = [c for _, c in spec]
    cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = int(cu[-1])
    rng = np.random.default_rng(P + 7)
    kn = rng.standard_normal((T, hkv, d)).astype(np.float32)
    vn = rng.standard_normal((T, hkv, d)).astype(np.float32)
    if kv_dtype == "bf16":
        kn, vn = bf16_bits(kn), bf16_bits(vn)
    ops = _ops()
    a, b = DeviceCase(case), DeviceCase(case)
    ws_a = ops.decode_plan(a.ctx, a.tables, hq, d, a.max_ctx, P)
    ws_b = ops.decode_plan(b.ctx, b.tables, hq, d, b.max_ctx, P)
    say(f"  append in pass {kv_dtype} P{P}")
    o1, l1 = ops.append_paged_decode_planned(a.q, a.k, a.v, dev(kn), dev(vn), a.tables,
                                             dev(start), dev(cu), a.ctx, a.max_ctx, ws_a,
                                             scale=float(case.scale), partition_size=P)
    ops.kv_append(b.k, b.v, dev(kn), dev(vn), b.tables, dev(start), dev(cu))
    o2, l2 = ops.paged_decode_planned(b.q, b.k, b.v, b.tables, b.ctx, b.max_ctx, ws_b,
                                      scale=float(case.scale), partition_size=P)
    torch.cuda.synchronize()
    assert a.k.cpu().numpy().tobytes() == b.k.cpu().numpy().tobytes()
    assert a.v.cpu().numpy().tobytes() == b.v.cpu().numpy().tobytes()
    assert o1.cpu().numpy().tobytes() == o2.cpu().numpy().tobytes()
    assert l1.cpu().numpy().tobytes() == l2.cpu().numpy().tobytes()
    kp, vp = pa.kv_append(case.k_pool[0], case.v_pool[0], kn, vn, case.block_tables, start, cu)
    want = pa.paged_decode(case.q[0], kp, vp, case.block_tables, case.context_lens, case.scale,
                           kv_dtype)
    assert_parity((o1.cpu().numpy(), l1.cpu().numpy()), want, kv_dtype, f"append in pass P{P}")
    assert_no_device_error()


def test_append_in_pass_over_layers_with_one_plan():
    """One plan per step, one launch per layer: every layer's pool and output equal the
    separate calls', and a position outside the table row is flagged like kv_append's."""
    case = config_case("qwen_gqa", 2, layers=3, max_batch=24)
    ops = _ops()
    si_start = (case.context_lens - 1).astype(np.int32)
    cu = np.arange(case.batch + 1, dtype=np.int32)
    rng = np.random.default_rng(11)
    P = 256
    plan = None
    for layer in range(3):
        kn = bf16_bits(rng.standard_normal((case.batch, case.num_kv_heads, case.head_dim))
                       .astype(np.float32))
        vn = bf16_bits(rng.standard_normal((case.batch, case.num_kv_heads, case.head_dim))
                       .astype(np.float32))
        a, b = DeviceCase(case, layer), DeviceCase(case, layer)
        if plan is None:
            plan = ops.decode_plan(a.ctx, a.tables, case.num_q_heads, case.head_dim, a.max_ctx, P)
        o1, l1 = ops.append_paged_decode_planned(a.q, a.k, a.v, dev(kn), dev(vn), a.tables,
                                                 dev(si_start), dev(cu), a.ctx, a.max_ctx, plan,
                                                 scale=float(case.scale), partition_size=P)
        o2, l2 = ops.append_paged_decode(b.q, b.k, b.v, dev(kn), dev(vn), b.tables,
                                         dev(si_start), dev(cu), b.ctx, b.max_ctx,
                                         scale=float(case.scale), partition_size=P)
        torch.cuda.synchronize()
        assert a.k.cpu().numpy().tobytes() == b.k.cpu().numpy().tobytes(), layer
        assert a.v.cpu().numpy().tobytes() == b.v.cpu().numpy().tobytes(), layer
        assert o1.cpu().numpy().tobytes() == o2.cpu().numpy().tobytes(), layer
        assert l1.cpu().numpy().tobytes() == l2.cpu().numpy().tobytes(), layer
    assert_no_device_error()
    # a position one past the table row: nothing is written, the position bit is set
    dc = DeviceCase(case)
    bad = si_start.copy()
    bad[3] = case.block_tables.shape[1] * 16
    before = dc.k.cpu().numpy().tobytes()
    ops.append_paged_decode_planned(dc.q, dc.k, dc.v, dev(kn), dev(vn), dc.tables, dev(bad),
                                    dev(cu), dc.ctx, dc.max_ctx, plan, scale=float(case.scale),
                                    partition_size=P)
    torch.cuda.synchronize()
    flags = ops.device_error()
    assert flags & 2, flags
    after = dc.k.cpu().numpy()
    assert after.tobytes() != before  # the other sequences' tokens were written


@pytest.mark.parametrize("shape", ["qwen_bf16_P256", "f32_d64_P0"])
def test_decode_step_layers_in_one_call(shape):
    """DecodeStep.layers (pkv_append_paged_decode_planned_layers: the step's layers stacked,
    one library call) leaves every layer's pool, out and lse equal to one layer() call per
    layer, bit for bit, with stacked outputs and with the bound one (the last layer's
    result); a stack whose layers do not match the first layer's is refused."""
    say(f"decode step layers: {shape}")
    if shape == "qwen_bf16_P256":
        case, P = config_case("qwen_gqa", 3, layers=4, max_batch=24), 256
    else:
        case = build_case("layers", [1, 16, 17, 300, 190, 33, 64, 2], 12, 12, 64, "f32",
                          seed=9, layers=4)
        P = 0
    ops = _ops()
    B, L = case.batch, 4
    conv = bf16_bits if case.kv_dtype == "bf16" else (lambda x: x)
    rng = np.random.default_rng(L)
    dims = (L, B, case.num_kv_heads, case.head_dim)
    kn = dev(conv(rng.standard_normal(dims).astype(np.float32)))
    vn = dev(conv(rng.standard_normal(dims).astype(np.float32)))
    start = dev((case.context_lens - 1).astype(np.int32))
    cu = dev(np.arange(B + 1, dtype=np.int32))
    tables, ctx = dev(case.block_tables), dev(case.context_lens)
    max_ctx = int(case.context_lens.max())
    q = dev(np.stack([case.q[l] for l in range(L)]))
    pools = [(dev(np.stack(case.k_pool[:L])), dev(np.stack(case.v_pool[:L]))) for _ in range(3)]
    steps = [ops.DecodeStep(q[0], pools[i][0][0], pools[i][1][0], kn[0], vn[0], tables, start,
                            cu, ctx, max_ctx, scale=float(case.scale), partition_size=P)
             for i in range(3)]
    outs = torch.empty((L, B, case.num_q_heads, case.head_dim), dtype=torch.float32,
                       device="cuda")
    lses = torch.empty((L, B, case.num_q_heads), dtype=torch.float32, device="cuda")
    ref = []
    for l in range(L):
        o, ls = steps[0].layer(q[l], pools[0][0][l], pools[0][1][l], kn[l], vn[l])
        ref.append((o.clone(), ls.clone()))
    steps[1].layers(q, pools[1][0], pools[1][1], kn, vn, out=outs, lse=lses)
    o_last, l_last = steps[2].layers(q, pools[2][0], pools[2][1], kn, vn)
    torch.cuda.synchronize()
    for i in (1, 2):
        assert pools[i][0].cpu().numpy().tobytes() == pools[0][0].cpu().numpy().tobytes(), i
        assert pools[i][1].cpu().numpy().tobytes() == pools[0][1].cpu().numpy().tobytes(), i
    for l in range(L):
        assert outs[l].cpu().numpy().tobytes() == ref[l][0].cpu().numpy().tobytes(), l
        assert lses[l].cpu().numpy().tobytes() == ref[l][1].cpu().numpy().tobytes(), l
    assert o_last.cpu().numpy().tobytes() == ref[-1][0].cpu().numpy().tobytes()
    assert l_last.cpu().numpy().tobytes() == ref[-1][1].cpu().numpy().tobytes()
    assert_no_device_error()
    with pytest.raises(ValueError):
        steps[1].layers(q[:, :-1], pools[1][0], pools[1][1], kn, vn)
    with pytest.raises(ValueError):
        steps[1].layers(q, pools[1][0][:3], pools[1][1], kn, vn)


@pytest.mark.parametrize("shape", ["qwen_bf16_P256", "f32_d64_P0"])
def test_append_paged_decode_layers_equals_decode_step(shape):
    """append_paged_decode_layers (plan + every layer, two library calls, the stacked
    tensors checked once) leaves pools, out and lse equal to DecodeStep.layers bit for
    bit; stacks that disagree are refused on the host."""
    say(f"append_paged_decode_layers: {shape}")
    if shape == "qwen_bf16_P256":
        case, P = config_case("qwen_gqa", 4, layers=3, max_batch=20), 256
    else:
        case = build_case("layers2", [1, 16, 17, 300, 190, 33], 12, 12, 64, "f32", seed=11,
                          layers=3)
        P = 0
    ops = _ops()
    B, L = case.batch, 3
    conv = bf16_bits if case.kv_dtype == "bf16" else (lambda x: x)
    rng = np.random.default_rng(17)
    dims = (L, B, case.num_kv_heads, case.head_dim)
    kn = dev(conv(rng.standard_normal(dims).astype(np.float32)))
    vn = dev(conv(rng.standard_normal(dims).astype(np.float32)))
    start = dev((case.context_lens - 1).astype(np.int32))
    cu = dev(np.arange(B + 1, dtype=np.int32))
    tables, ctx = dev(case.block_tables), dev(case.context_lens)
    max_ctx = int(case.context_lens.max())
    q = dev(np.stack([case.q[l] for l in range(L)]))
    pools = [(dev(np.stack(case.k_pool[:L])), dev(np.stack(case.v_pool[:L]))) for _ in range(2)]
    outs = [torch.empty((L, B, case.num_q_heads, case.head_dim), dtype=torch.float32,
                        device="cuda") for _ in range(2)]
    lses = [torch.empty((L, B, case.num_q_heads), dtype=torch.float32, device="cuda")
            for _ in range(2)]
    step = ops.DecodeStep(q[0], pools[0][0][0], pools[0][1][0], kn[0], vn[0], tables, start, cu,
                          ctx, max_ctx, scale=float(case.scale), partition_size=P)
    step.layers(q, pools[0][0], pools[0][1], kn, vn, out=outs[0], lse=lses[0])
    ws = torch.empty(ops.decode_workspace_bytes(B, case.num_q_heads, case.head_dim, max_ctx, P),
                     dtype=torch.uint8, device="cuda")
    ops.append_paged_decode_layers(q, pools[1][0], pools[1][1], kn, vn, tables, start, cu, ctx,
                                   max_ctx, ws, scale=float(case.scale), partition_size=P,
                                   out=outs[1], lse=lses[1])
    torch.cuda.synchronize()
    for a, b in ((pools[0][0], pools[1][0]), (pools[0][1], pools[1][1]), (outs[0], outs[1]),
                 (lses[0], lses[1])):
        assert a.cpu().numpy().tobytes() == b.cpu().numpy().tobytes()
    assert_no_device_error()
    with pytest.raises(ValueError):
        ops.append_paged_decode_layers(q[:2], pools[1][0], pools[1][1], kn, vn, tables, start,
                                       cu, ctx, max_ctx, ws, partition_size=P, out=outs[1][0])
    with pytest.raises(ValueError):
        ops.append_paged_decode_layers(q, pools[1][0], pools[1][1], kn, vn, tables, start, cu,
                                       ctx, max_ctx, ws, partition_size=P, out=outs[1][:, :-1])


@pytest.mark.parametrize("shape", ["qwen_bf16_P256", "f32_d128_P0"])
def test_decode_step_equals_planned_calls(shape):
    """DecodeStep (step-wide tensors bound and planned once, one layer() per layer) leaves
    every layer's pool, out and lse equal to append_paged_decode_planned's, bit for bit;
    after context lengths and positions change in place, plan() re-plans for them."""
    say(f"decode step: {shape}, 3 layers, 2 steps")
    if shape == "qwen_bf16_P256":
        case, P = config_case("qwen_gqa", 2, layers=3, max_batch=24), 256
    else:
        case = build_case("step", [1, 16, 17, 300, 1000, 33, 64, 2], 16, 4, 128, "f32", seed=8,
                          layers=3)
        P = 0
    ops = _ops()
    B = case.batch
    start = dev((case.context_lens - 1).astype(np.int32))
    cu = dev(np.arange(B + 1, dtype=np.int32))
    rng = np.random.default_rng(5)
    a = [DeviceCase(case, layer) for layer in range(3)]
    b = [DeviceCase(case, layer) for layer in range(3)]
    ctx_a, ctx_b = a[0].ctx.clone(), b[0].ctx.clone()
    tables = a[0].tables
    news = []
    conv = bf16_bits if case.kv_dtype == "bf16" else (lambda x: x)
    for _ in range(6):
        dims = (B, case.num_kv_heads, case.head_dim)
        news.append((dev(conv(rng.standard_normal(dims).astype(np.float32))),
                     dev(conv(rng.standard_normal(dims).astype(np.float32)))))
    outs = [torch.empty((B, case.num_q_heads, case.head_dim), dtype=torch.float32,
                        device="cuda") for _ in range(3)]
    step = ops.DecodeStep(a[0].q, a[0].k, a[0].v, *news[0], tables, start, cu, ctx_a,
                          a[0].max_ctx, scale=float(case.scale), partition_size=P)
    for it in range(2):
        if it == 1:
            # the next step: shorter contexts, each new token at its sequence's last slot
            shorter = torch.clamp(ctx_a - 3, min=1)
            ctx_a.copy_(shorter)
            ctx_b.copy_(shorter)
            start.copy_(shorter - 1)
            step.plan()
        plan = ops.decode_plan(ctx_b, tables, case.num_q_heads, case.head_dim, b[0].max_ctx, P)
        for layer in range(3):
            kn, vn = news[3 * it + layer]
            # layer 1 writes into its own output buffer, the others into the bound one
            o1, l1 = step.layer(a[layer].q, a[layer].k, a[layer].v, kn, vn,
                                out=outs[layer] if layer == 1 else None)
            o1, l1 = o1.clone(), l1.clone()
            o2, l2 = ops.append_paged_decode_planned(b[layer].q, b[layer].k, b[layer].v, kn, vn,
                                                     tables, start, cu, ctx_b, b[0].max_ctx,
                                                     plan, scale=float(case.scale),
                                                     partition_size=P)
            torch.cuda.synchronize()
            tag = (it, layer)
            assert a[layer].k.cpu().numpy().tobytes() == b[layer].k.cpu().numpy().tobytes(), tag
            assert a[layer].v.cpu().numpy().tobytes() == b[layer].v.cpu().numpy().tobytes(), tag
            assert o1.cpu().numpy().tobytes() == o2.cpu().numpy().tobytes(), tag
            assert l1.cpu().numpy().tobytes() == l2.cpu().numpy().tobytes(), tag
    assert_no_device_error()
    # a layer whose tensors do not match the first layer's is refused on the host
    with pytest.raises(ValueError):
        step.layer(a[0].q[:-1], a[0].k, a[0].v, *news[0])
    with pytest.raises(ValueError):
        step.layer(a[0].q, a[0].k.half(), a[0].v, *news[0])
    with pytest.raises(ValueError):
        step.layer(a[0].q, a[0].k, a[0].v, news[0][0].cpu(), news[0][1])
