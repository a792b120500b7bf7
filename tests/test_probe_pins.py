"""The one-hot gather probes, pinned on the CPU: for probe inputs the float64 oracle's
attention, rounded to float32, is exactly the hot key's V row, for plain decode, split
partitions merged by log-sum-exp, copy-on-write forks and chunked prefill.  So a GPU
result equal to the probe's expected rows is equal to the oracle rounded to float32, value
for value.  (Only a zero's sign is left open: where the hot value is 0 the oracle's sign is
that of a ~1e-70 remainder.)  Planted indexing mistakes (a table off by one block, a wrong
KV head, a causal limit one token too far, a length one too short) change the result, so
the probes can see them."""

from __future__ import annotations

import numpy as np
import pytest

import oracle.paged_attention as pa
import oracle.paged_prefill as pp
from probe_util import (check_decode_hot, decode_expected, decode_probe, decode_round_q,
                        decode_rounds, fork_probe, prefill_expected, prefill_probe, v_rows)
from workloads import build_case, fork_case, fork_groups


def _as32(x):
    return np.asarray(x, np.float64).astype(np.float32)


@pytest.mark.parametrize("kv_dtype,hq,hkv,d", [("bf16", 8, 2, 16), ("f32", 6, 6, 8),
                                               ("bf16", 7, 1, 8), ("f32", 4, 2, 32)])
def test_decode_probe_is_the_oracle(kv_dtype, hq, hkv, d):
    lens = [1, 5, 16, 17, 40, 0, 97]
    case = build_case("pin", lens, hq, hkv, d, kv_dtype, seed=hq + d)
    case.scale = np.float32(1.0)
    phases = -(-max(-(-n // 16) for n in lens) // (hkv * d))
    for phase in range(max(1, phases)):
        hot = decode_probe(case, 0, phase, seed=phase)
        check_decode_hot(case, hot)
        vseq = v_rows(case.v_pool[0], case.block_tables, case.context_lens, kv_dtype)
        for r in range(decode_rounds(hq, hkv, d)):
            q, dims = decode_round_q(case.batch, hq, hkv, d, r, kv_dtype)
            want = decode_expected(vseq, hot, hq, dims)
            o, l = pa.paged_decode(q, case.k_pool[0], case.v_pool[0], case.block_tables,
                                   case.context_lens, case.scale, kv_dtype)
            assert np.array_equal(_as32(o), want), f"round {r}"
            # split into partitions of 16 and 32 tokens and merged: the same bits
            for P in (16, 32):
                po, pl = pa.decode_partitions(q, case.k_pool[0], case.v_pool[0],
                                              case.block_tables, case.context_lens, case.scale,
                                              kv_dtype, P)
                co, cl = pa.combine_partitions(po, pl)
                assert np.array_equal(_as32(co), want), f"round {r} P{P}"


def test_decode_probe_sees_indexing_mistakes():
    case = build_case("pin", [40, 97, 33], 8, 2, 16, "bf16", seed=3)
    case.scale = np.float32(1.0)
    hot = decode_probe(case, 0, 0, seed=1)
    vseq = v_rows(case.v_pool[0], case.block_tables, case.context_lens, "bf16")
    q, dims = decode_round_q(case.batch, 8, 2, 16, 0, "bf16")
    want = decode_expected(vseq, hot, 8, dims)
    # block ids read one logical block late
    t2 = case.block_tables.copy()
    t2[:, :-1] = case.block_tables[:, 1:]
    o, _ = pa.paged_decode(q, case.k_pool[0], case.v_pool[0], t2, case.context_lens,
                           case.scale, "bf16")
    assert not np.array_equal(_as32(o), want)
    # one token short of the explicit length (the newest token is dimension 0's hot key)
    o, _ = pa.paged_decode(q, case.k_pool[0], case.v_pool[0], case.block_tables,
                           case.context_lens - 1, case.scale, "bf16")
    assert not np.array_equal(_as32(o), want)
    # KV heads swapped
    o, _ = pa.paged_decode(q, case.k_pool[0][:, ::-1].copy(), case.v_pool[0],
                           case.block_tables, case.context_lens, case.scale, "bf16")
    assert not np.array_equal(_as32(o), want)


@pytest.mark.parametrize("kv_dtype", ["bf16", "f32"])
def test_fork_probe_is_the_oracle(kv_dtype):
    case = fork_case("pin", [32, 48, 20], 3, [[0, 5, 17], [16, 0, 1], [0, 0, 0]], 4, 2, 16,
                     kv_dtype, seed=5)
    case.scale = np.float32(1.0)
    gs, gb = fork_groups(case)
    hot = fork_probe(case, gs, gb, 0, seed=2)
    check_decode_hot(case, hot)
    vseq = v_rows(case.v_pool[0], case.block_tables, case.context_lens, kv_dtype)
    for r in range(decode_rounds(4, 2, 16)):
        q, dims = decode_round_q(case.batch, 4, 2, 16, r, kv_dtype)
        want = decode_expected(vseq, hot, 4, dims)
        o, _ = pa.paged_decode(q, case.k_pool[0], case.v_pool[0], case.block_tables,
                               case.context_lens, case.scale, kv_dtype)
        assert np.array_equal(_as32(o), want), f"round {r}"


def _prefill_probe_case(kv_dtype, hq, hkv, d, lens, chunks, seed):
    case = build_case("pin", lens, hq, hkv, d, kv_dtype, seed=seed)
    case.scale = np.float32(1.0)
    cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    start = (np.asarray(lens) - np.asarray(chunks)).astype(np.int32)
    q, hot = prefill_probe(case, None, cu, start, 0, seed=seed)
    return case, cu, q, hot


@pytest.mark.parametrize("kv_dtype,hq,hkv,d", [("bf16", 8, 2, 16), ("f32", 3, 3, 8),
                                               ("bf16", 7, 1, 8)])
def test_prefill_probe_is_the_oracle(kv_dtype, hq, hkv, d):
    lens, chunks = [40, 17, 60, 9], [40, 3, 25, 0]
    case, cu, q, hot = _prefill_probe_case(kv_dtype, hq, hkv, d, lens, chunks, seed=hq)
    vseq = v_rows(case.v_pool[0], case.block_tables, case.context_lens, kv_dtype)
    want = prefill_expected(vseq, hot, cu, hq, hkv)
    o, _ = pp.paged_prefill(q, case.k_pool[0], case.v_pool[0], case.block_tables, cu,
                            case.context_lens, case.scale, kv_dtype)
    assert np.array_equal(_as32(o), want)


def test_prefill_probe_sees_a_causal_limit_one_token_too_far():
    lens, chunks = [40, 60], [40, 25]
    case, cu, q, hot = _prefill_probe_case("bf16", 8, 2, 16, lens, chunks, seed=4)
    vseq = v_rows(case.v_pool[0], case.block_tables, case.context_lens, "bf16")
    want = prefill_expected(vseq, hot, cu, 8, 2)
    # sequence 0's first 39 queries given as a chunk of 39 in its 40-token context: query
    # i then sits at position i + 1, one token past its own limit
    o, _ = pp.paged_prefill(q[:39], case.k_pool[0], case.v_pool[0], case.block_tables[:1],
                            np.array([0, 39], np.int32), case.context_lens[:1], case.scale,
                            "bf16")
    assert not np.array_equal(_as32(o), want[:39])
    # and at the right positions they are the expected rows
    o, _ = pp.paged_prefill(q[:40], case.k_pool[0], case.v_pool[0], case.block_tables[:1],
                            np.array([0, 40], np.int32), case.context_lens[:1], case.scale,
                            "bf16")
    assert np.array_equal(_as32(o), want[:40])
