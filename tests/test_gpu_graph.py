"""Library calls captured in a HIP graph (torch.cuda.CUDAGraph) replay to the eager
results, bit for bit, on every replay, with eager work and synchronisations between
replays: multi-layer append + decode (per-layer calls and DecodeStep), the shared-prefix decode
and the prefill."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_util import assert_no_device_error, dev, say
from libpkv_util import ensure_built
from workloads import bf16_bits, chunked_prefill_case, config_case, fork_groups

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ensure_built()


def _check_graph(step, outputs, replays=3):
    """Eager result, then capture; every replay must reproduce it bit for bit."""
    step()
    torch.cuda.synchronize()
    want = [o.clone() for o in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(replays):
        for o in outputs:
            o.fill_(float("nan"))            # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outputs, want):
            assert torch.equal(o, w), f"replay {r} differs from the eager result"
    assert_no_device_error()


def test_graph_multilayer_append_decode():
    import paged_kv_cache_200_amd as pkv
    say("graph: 4-layer append + decode, Qwen shape")
    case = config_case("qwen_gqa", 0, layers=4)
    B, hq, hkv, d = case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim
    qs = [dev(case.q[l]) for l in range(4)]
    ks = [dev(case.k_pool[l]) for l in range(4)]
    vs = [dev(case.v_pool[l]) for l in range(4)]
    tables, ctx = dev(case.block_tables), dev(case.context_lens)
    mx = int(case.context_lens.max())
    rng = np.random.default_rng(3)
    kn = dev(bf16_bits(rng.standard_normal((B, hkv, d)).astype(np.float32)))
    vn = dev(bf16_bits(rng.standard_normal((B, hkv, d)).astype(np.float32)))
    start = dev((case.context_lens - 1).astype(np.int32))
    cu = dev(np.arange(B + 1, dtype=np.int32))
    outs = [torch.empty((B, hq, d), dtype=torch.float32, device="cuda") for _ in range(4)]
    lses = [torch.empty((B, hq), dtype=torch.float32, device="cuda") for _ in range(4)]
    ws = torch.empty(pkv.decode_workspace_bytes(B, hq, d, mx, 512), dtype=torch.uint8,
                     device="cuda")

    def step():
        for l in range(4):
            pkv.append_paged_decode(qs[l], ks[l], vs[l], kn, vn, tables, start, cu, ctx, mx,
                                    scale=float(case.scale), partition_size=512, out=outs[l],
                                    lse=lses[l], workspace=ws)

    _check_graph(step, outs + lses)


def test_graph_shared_prefix_decode():
    import paged_kv_cache_200_amd as pkv
    say("graph: shared-prefix decode, fork workload")
    case = config_case("prefix_fork", 0)
    B, hq, d = case.batch, case.num_q_heads, case.head_dim
    gs, gb = fork_groups(case)
    mx = int(case.context_lens.max())
    q, k, v = dev(case.q[0]), dev(case.k_pool[0]), dev(case.v_pool[0])
    tables, ctx = dev(case.block_tables), dev(case.context_lens)
    out = torch.empty((B, hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, hq), dtype=torch.float32, device="cuda")
    ws = torch.empty(pkv.shared_prefix_workspace_bytes(B, hq, d, mx, 1024), dtype=torch.uint8,
                     device="cuda")
    dgs, dgb = dev(gs), dev(gb)

    def step():
        pkv.paged_decode_shared_prefix(q, k, v, tables, ctx, dgs, dgb, int(gb.max()), mx,
                                       scale=float(case.scale), partition_size=1024, out=out,
                                       lse=lse, workspace=ws)

    _check_graph(step, [out, lse])


def test_graph_prefill():
    import paged_kv_cache_200_amd as pkv
    say("graph: chunked prefill")
    pc = chunked_prefill_case(0, batch=4, chunk=128, max_prior=512)
    case = pc.case
    T = int(pc.cu_q[-1])
    q, k, v = dev(pc.q), dev(case.k_pool[0]), dev(case.v_pool[0])
    tables, ctx, cu = dev(case.block_tables), dev(case.context_lens), dev(pc.cu_q)
    out = torch.empty((T, case.num_q_heads, case.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, case.num_q_heads), dtype=torch.float32, device="cuda")

    def step():
        pkv.paged_prefill(q, k, v, tables, cu, ctx, 128, scale=float(case.scale), out=out,
                          lse=lse)

    _check_graph(step, [out, lse])


def test_graph_decode_step():
    """One plan per step and one launch per layer (DecodeStep), captured whole."""
    import paged_kv_cache_200_amd as pkv
    say("graph: DecodeStep, plan + 4 layers, Qwen shape")
    case = config_case("qwen_gqa", 1, layers=4)
    B, hq, hkv, d = case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim
    qs = [dev(case.q[l]) for l in range(4)]
    ks = [dev(case.k_pool[l]) for l in range(4)]
    vs = [dev(case.v_pool[l]) for l in range(4)]
    tables, ctx = dev(case.block_tables), dev(case.context_lens)
    mx = int(case.context_lens.max())
    rng = np.random.default_rng(4)
    kn = dev(bf16_bits(rng.standard_normal((B, hkv, d)).astype(np.float32)))
    vn = dev(bf16_bits(rng.standard_normal((B, hkv, d)).astype(np.float32)))
    start = dev((case.context_lens - 1).astype(np.int32))
    cu = dev(np.arange(B + 1, dtype=np.int32))
    outs = [torch.empty((B, hq, d), dtype=torch.float32, device="cuda") for _ in range(4)]
    lses = [torch.empty((B, hq), dtype=torch.float32, device="cuda") for _ in range(4)]
    ds = pkv.DecodeStep(qs[0], ks[0], vs[0], kn, vn, tables, start, cu, ctx, mx,
                        scale=float(case.scale), partition_size=256, plan=False)

    def step():
        ds.plan()
        for l in range(4):
            ds.layer(qs[l], ks[l], vs[l], kn, vn, out=outs[l], lse=lses[l])

    _check_graph(step, outs + lses)
