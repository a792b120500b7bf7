"""The exact library calls bench.py times, at the workloads' full sizes, against the oracle:
the 256-sequence decode step (append + decode in one call, at the library's partition-size
rule and at partition 4096), the
copy-on-write fork step (append + shared-prefix decode, partition 1024) and the chunked
prefill (every sequence, sampled query rows)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_util import assert_no_device_error, assert_parity, dev, say
from libpkv_util import ensure_built
from oracle import paged_attention as pa
from oracle import paged_prefill as pp
from workloads import chunked_prefill_case, config_case, decode_step_inputs, fork_groups

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ensure_built()


def _oracle_step(case, si):
    kp, vp = pa.kv_append(case.k_pool[0], case.v_pool[0], si.k_new, si.v_new,
                          case.block_tables, si.start_pos, si.cu_new)
    return pa.paged_decode(case.q[0], kp, vp, case.block_tables, case.context_lens, case.scale,
                           case.kv_dtype)


@pytest.mark.parametrize("seed,rule", [(0, True), (1, True), (2, True), (0, False), (1, False)])
def test_high_concurrency_step_as_benched(seed, rule):
    """Seeds 0-2 at the rule's partition size; at 4096, seed 1 holds an 8192-token
    sequence, exactly two full partitions."""
    import paged_kv_cache_200_amd as pkv
    case = config_case("high_concurrency", seed)
    P = (pkv.decode_partition_size(case.batch, 8, 128, int(case.context_lens.max()),
                                   int(case.context_lens.sum())) if rule else 4096)
    say(f"bench config: high_concurrency seed {seed}, append_paged_decode, P={P}")
    si = decode_step_inputs(case, seed)
    k, v = dev(case.k_pool[0]), dev(case.v_pool[0])
    o, l = pkv.append_paged_decode(dev(case.q[0]), k, v, dev(si.k_new), dev(si.v_new),
                                   dev(case.block_tables), dev(si.start_pos), dev(si.cu_new),
                                   dev(case.context_lens), int(case.context_lens.max()),
                                   scale=float(case.scale), partition_size=P)
    torch.cuda.synchronize()
    kp, vp = pa.kv_append(case.k_pool[0], case.v_pool[0], si.k_new, si.v_new,
                          case.block_tables, si.start_pos, si.cu_new)
    assert k.cpu().numpy().tobytes() == kp.tobytes(), "K pool after the append"
    assert v.cpu().numpy().tobytes() == vp.tobytes(), "V pool after the append"
    assert_parity((o.cpu().numpy(), l.cpu().numpy()),
                  pa.paged_decode(case.q[0], kp, vp, case.block_tables, case.context_lens,
                                  case.scale, case.kv_dtype),
                  "bf16", f"high_concurrency s{seed} P{P} as benched")
    assert_no_device_error()


def test_prefix_fork_step_as_benched():
    import paged_kv_cache_200_amd as pkv
    say("bench config: prefix_fork, append_paged_decode_shared_prefix, P=1024")
    case = config_case("prefix_fork", 0)
    si = decode_step_inputs(case, 0)
    assert si.cu_new[-1] < case.batch  # forks with no private token append nothing
    gs, gb = fork_groups(case)
    o, l = pkv.append_paged_decode_shared_prefix(
        dev(case.q[0]), dev(case.k_pool[0]), dev(case.v_pool[0]), dev(si.k_new), dev(si.v_new),
        dev(case.block_tables), dev(si.start_pos), dev(si.cu_new), dev(case.context_lens),
        dev(gs), dev(gb), int(gb.max()), int(case.context_lens.max()),
        scale=float(case.scale), partition_size=1024)
    torch.cuda.synchronize()
    assert_parity((o.cpu().numpy(), l.cpu().numpy()), _oracle_step(case, si), "bf16",
                  "prefix_fork as benched")
    assert_no_device_error()


def test_chunked_prefill_as_benched():
    import paged_kv_cache_200_amd as pkv
    say("bench config: chunked_prefill, kv_append + paged_prefill, every sequence")
    pc = chunked_prefill_case(0)
    case = pc.case
    k, v = dev(case.k_pool[0]), dev(case.v_pool[0])
    tables, ctx, cu = dev(case.block_tables), dev(case.context_lens), dev(pc.cu_q)
    pkv.kv_append(k, v, dev(pc.k_new), dev(pc.v_new), tables, dev(pc.start_pos), cu)
    o, l = pkv.paged_prefill(dev(pc.q), k, v, tables, cu, ctx, int(np.diff(pc.cu_q).max()),
                             scale=float(case.scale))
    torch.cuda.synchronize()
    o, l = o.cpu().numpy(), l.cpu().numpy()
    kp, vp = pa.kv_append(case.k_pool[0], case.v_pool[0], pc.k_new, pc.v_new,
                          case.block_tables, pc.start_pos, pc.cu_q)
    # every sequence; of each chunk the first and last four query rows and 24 drawn ones.
    # Query i of a chunk of L at context n attends tokens [0, n - L + i]: the oracle takes
    # it as a one-token chunk of the context cut to n - L + i + 1 tokens.
    rng = np.random.default_rng(0)
    for s in range(case.batch):
        r0, r1 = int(pc.cu_q[s]), int(pc.cu_q[s + 1])
        L, n = r1 - r0, int(case.context_lens[s])
        rows = sorted(set(range(4)) | set(range(L - 4, L)) | set(rng.integers(0, L, 24).tolist()))
        got_o, got_l, want_o, want_l = [], [], [], []
        for i in rows:
            wo, wl = pp.paged_prefill(pc.q[r0 + i:r0 + i + 1], kp, vp, case.block_tables[s:s + 1],
                                      np.array([0, 1], np.int32),
                                      np.array([n - L + i + 1], np.int32), case.scale, "bf16")
            got_o.append(o[r0 + i]); got_l.append(l[r0 + i])
            want_o.append(wo[0]); want_l.append(wl[0])
        assert_parity((np.array(got_o), np.array(got_l)), (np.array(want_o), np.array(want_l)),
                      "bf16", f"chunked prefill seq {s} ({len(rows)} rows)")
    assert_no_device_error()
