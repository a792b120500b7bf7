#!/usr/bin/env python3
"""Paged decode attention benchmark on one MI355X.

One step = the whole decode hot path over one batch: KV append of each
sequence's new token at its explicit position, then paged decode attention
(split-KV first pass + log-sum-exp combine) over the block-paged cache.

Default workload: 256 sequences, bf16 K/V, 32 query heads over 8 KV heads,
head_dim 128, block size 16, context lengths lognormal (median 1024, max
8192), blocks randomly scattered over a pool of 1.2x the tokens (seeded,
synthetic).  Inputs are resident in HBM before the timed region.

Prints one JSON line.  ``value`` is the step's achieved HBM throughput in GB/s
from algorithmic bytes (K/V of every attended token, q, out, lse, block-table
entries, lengths, and the appended rows).  ``roofline`` is the first-pass
kernel alone, timed with HIP events on the stream it runs on.
``cpu_baseline`` is the float64 CPU oracle on the same inputs.
"""

from __future__ import annotations

import argparse
import gc
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# a step whose bytes fit the MI355X's 256 MB Infinity Cache is also timed cold
INFINITY_CACHE_BYTES = 256 << 20
# HBM traffic records (rocprofv3 counters) of the first pass, per workload
TRAFFIC_FILES = {w: os.path.join(ROOT, "profiles", f"traffic_{w}.json")
                 for w in ("high_concurrency", "long_context", "qwen_gqa")}
# the sources that define the first pass (and the plan/append prologue of its step);
# counters taken on other sources are not reported
DECODE_SRCS = [os.path.join(ROOT, "paged_kv_cache_200_amd", "csrc", f)
               for f in ("paged_decode.hip", "common.h", "append_row.h", "valu_attend.h",
                         "mfma_tile.h")]


def decode_source_digest():
    """SHA-256 of the first pass's code: its sources without // comments, trailing blanks
    and empty lines, so that editing a comment keeps the counters taken on that code."""
    h = hashlib.sha256()
    for path in DECODE_SRCS:
        for line in open(path, encoding="utf-8").read().splitlines():
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="high_concurrency",
                   choices=["high_concurrency", "long_context", "prefix_fork", "qwen_gqa", "tiny",
                            "gpt2_replay", "chunked_prefill"])
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--partition-size", type=int, default=None,
                   help="split-KV partition size in tokens (default: the workload's own, else "
                        "1024 for fork groups on the shared-prefix path, else 4096)")
    p.add_argument("--kernel-reps", type=int, default=50)
    p.add_argument("--settle-seconds", type=float, default=0.3,
                   help="before the warmup steps, run steps (untimed) for this long: the GPU's "
                        "clocks take a few hundred ms of load to settle, far longer than a few "
                        "0.2 ms warmup steps")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="target CPU time for the oracle baseline (repeats the whole batch)")
    p.add_argument("--no-copy-probe", action="store_true")
    p.add_argument("--graph", action="store_true",
                   help="replay the step as one captured HIP graph instead of launching "
                        "every library call from Python (measured no faster here)")
    p.add_argument("--decode-path", choices=["valu", "mfma"], default="valu",
                   help="plain (non-fork) workloads: valu = the first pass (default); mfma = "
                        "the matrix-core tile of the shared-prefix path with every sequence a "
                        "group of one (the dense-tile variant, for comparison)")
    p.add_argument("--crossover", action="store_true",
                   help="instead of one workload: sweep batch x context x partition size on "
                        "uniform-length bf16 workloads (32/8 heads, head_dim 128) and print "
                        "where splitting the KV length pays")
    p.add_argument("--no-shared-prefix", action="store_true",
                   help="decode fork workloads with the plain path (each fork re-reads the "
                        "shared prefix) instead of the shared-prefix path")
    p.add_argument("--append-in-pass", choices=["auto", "yes", "no"], default="auto",
                   help="plain decode: one work plan per step, then one launch per layer that "
                        "appends the new tokens and attends (pkv_append_paged_decode_planned), "
                        "instead of a plan + append launch and a first-pass launch per layer; "
                        "auto: when the step has more than one layer (measured faster there, "
                        "3 us slower on one layer)")
    p.add_argument("--cold", action="store_true",
                   help="read a 1 GiB scratch buffer before every timed step (outside the "
                        "timed region), so no step finds the previous one's data in the L2 "
                        "or the 256 MB Infinity Cache; each step is then timed on its own")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="before the timed steps, run 3 device copies of MIB MiB (a known-size "
                        "reference for HBM traffic counters)")
    return p.parse_args()


def settle(fn, torch, seconds):
    """Run fn, untimed, until `seconds` of wall time have passed."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def algorithmic_bytes(case, append_tokens: int):
    """Bytes the decode path must move: (decode, append)."""
    eb = case.elem_bytes
    B, hq, hkv, d = case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim
    ctx = case.context_lens.astype("int64")
    kv = int(ctx.sum()) * 2 * hkv * d * eb
    per_seq = B * (hq * d * eb + hq * d * 4 + hq * 4 + 4) + int(((ctx + 15) // 16).sum()) * 4
    decode = kv + per_seq
    # append: read k_new/v_new, write the cache rows, start_pos + cu + one table entry each
    append = append_tokens * (2 * 2 * hkv * d * eb + 4 * 3)
    return decode, append


def copy_probe(torch, nbytes=2 << 30, reps=10):
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1.0)
    b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    sec = s.elapsed_time(e) / 1e3 / reps
    del a, b
    return 2 * nbytes / sec / 1e9


def traffic_from_profile(workload, partition_size, seed):
    """HBM bytes per launch from committed PMC counters, if taken on this kernel source,
    workload, partition size and seed."""
    path = TRAFFIC_FILES.get(workload)
    if path is None:
        return None
    try:
        info = json.load(open(path))
    except (OSError, ValueError):
        return None
    if (info.get("kernel_source_sha256") == decode_source_digest()
            and info.get("partition_size") == partition_size and info.get("seed") == seed):
        return info.get("bytes_per_launch")
    return None


def cpu_baseline(case, decode_bytes, target_s):
    import numpy as np  # noqa: F401
    import oracle.paged_attention as pa
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    reps, t_total = 0, 0.0
    while reps == 0 or (t_total < target_s and reps < 5):
        t0 = time.perf_counter()
        pa.paged_decode(case.q[0], case.k_pool[0], case.v_pool[0], case.block_tables,
                        case.context_lens, case.scale, case.kv_dtype)
        t_total += time.perf_counter() - t0
        reps += 1
    sec = t_total / reps
    return {
        "value": round(decode_bytes / sec / 1e9, 3),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"whole {case.name} batch, layer 0 ({case.batch} sequences, sum ctx "
                   f"{int(case.context_lens.sum())}), decode only, float64 numpy, {reps} rep(s), "
                   f"{sec:.2f} s each; host affinity {len(os.sched_getaffinity(0))} cpus"),
        "seq_tokens_per_s": round(float(case.context_lens.sum()) / sec, 1),
    }


def unique_kv_tokens(case):
    """Tokens whose K/V must come from HBM at least once: each physical block counted
    once, with the largest number of valid slots any sequence uses in it."""
    valid = {}
    for s, n in enumerate(case.context_lens.tolist()):
        for j in range(-(-n // 16)):
            b = int(case.block_tables[s, j])
            valid[b] = max(valid.get(b, 0), min(16, n - 16 * j))
    return sum(valid.values())


MFMA_BF16_PEAK_TFLOPS = 2500.0


def run_prefill(args, np, torch, pkv):
    """Chunked prefill: append each sequence's 512-token chunk, then attend it causally
    over the whole context (one library call each), on the matrix cores (bf16)."""
    from workloads import chunked_prefill_case
    print(f"[bench] building inputs: chunked_prefill seed {args.seed}", file=sys.stderr,
          flush=True)
    pc = chunked_prefill_case(args.seed)
    case = pc.case
    B, hq, hkv, d = case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim

    def to_dev(x):
        if x.dtype == np.uint16:
            x = x.view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()

    kc, vc = to_dev(case.k_pool[0]), to_dev(case.v_pool[0])
    tables, ctx = to_dev(case.block_tables), to_dev(case.context_lens)
    q, k_new, v_new = to_dev(pc.q), to_dev(pc.k_new), to_dev(pc.v_new)
    cu, start = to_dev(pc.cu_q), to_dev(pc.start_pos)
    T = int(pc.cu_q[-1])
    max_q = int(np.diff(pc.cu_q).max())
    out = torch.empty((T, hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, hq), dtype=torch.float32, device="cuda")
    scale = float(case.scale)

    def prefill():
        pkv.paged_prefill(q, kc, vc, tables, cu, ctx, max_q, scale=scale, out=out, lse=lse)

    def step():
        pkv.kv_append(kc, vc, k_new, v_new, tables, start, cu)
        prefill()

    settle(step, torch, args.settle_seconds)
    for _ in range(args.warmup):
        step()
    stream = torch.cuda.current_stream()
    s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s_ev.record(stream)
    for _ in range(args.steps):
        step()
    e_ev.record(stream)
    torch.cuda.synchronize()
    step_s = s_ev.elapsed_time(e_ev) / 1e3 / args.steps
    s_ev.record(stream)
    for _ in range(args.kernel_reps):
        prefill()
    e_ev.record(stream)
    torch.cuda.synchronize()
    kern_s = s_ev.elapsed_time(e_ev) / 1e3 / args.kernel_reps
    # the error word is read after the timed launches (the read waits on the GPU)
    flags = pkv.device_error()
    if flags:
        raise RuntimeError(f"device error: {pkv.describe_device_error(flags)}")
    # causal work: query i of a chunk of L at context n attends n - L + i + 1 keys; per key
    # and query head 2 D flops for the score and 2 D for the weighted sum
    keys = 0
    for s in range(B):
        n, L = int(case.context_lens[s]), int(pc.cu_q[s + 1] - pc.cu_q[s])
        keys += L * (n - L) + L * (L + 1) // 2
    flops = keys * hq * d * 4
    kv_bytes = int(case.context_lens.sum()) * 2 * hkv * d * case.elem_bytes
    io_bytes = T * hq * d * (case.elem_bytes + 4) + T * hq * 4
    tflops = flops / kern_s / 1e12
    return {
        "metric": "paged chunked-prefill attention TFLOP/s at 1 GPU",
        "value": round(flops / step_s / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": args.settle_seconds,
        "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "chunked_prefill", "seed": args.seed, "batch": B,
                   "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": d, "block_size": 16,
                   "chunk_tokens": max_q, "sum_context_tokens": int(case.context_lens.sum()),
                   "query_tokens": T,
                   "step": "kv_append of the chunks + paged prefill (one launch each)"},
        "query_tokens_per_s": round(T / step_s, 1),
        "flops_per_step": flops,
        "roofline": {
            "kernel": "prefill_t32_kernel",
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None,
            "avg_launch_us": round(kern_s * 1e6, 2),
            "kv_bytes_per_launch": kv_bytes + io_bytes,
            "kv_gbps_if_read_once": round((kv_bytes + io_bytes) / kern_s / 1e9, 1),
        },
        "cpu_baseline": None,
    }


def run_replay(args, np, torch, pkv):
    """The GPT-2-shaped continuous-batching replay, end to end (host block manager,
    table uploads and every layer's append + decode), timed on the wall clock."""
    from workloads import replay_schedule, replay_step_values
    sched = replay_schedule(args.seed)
    L, hq, hkv, d, nb, bs = (sched.layers, sched.num_q_heads, sched.num_kv_heads, sched.head_dim,
                             sched.num_blocks, sched.block_size)
    W = -(-(128 + 192) // bs)
    kc = torch.zeros((L, nb, hkv, bs, d), dtype=torch.float32, device="cuda")
    vc = torch.zeros_like(kc)
    B = sched.batch
    steps = sched.steps
    # every step's inputs are drawn and uploaded before the timed region
    q_all, kv_all, plan = [], [], []
    for t in range(steps):
        active = [s for s in range(B) if t < int(sched.gen_lens[s])]
        plan.append(active)
        # the step's layers stacked: q [L, n, hq, d], new K and V [L, n, hkv, d]
        q_all.append(torch.from_numpy(np.stack(
            [replay_step_values(sched, t, l, active, "q") for l in range(L)])).cuda())
        kv = [replay_step_values(sched, t, l, active, "kv") for l in range(L)]
        kv_all.append(tuple(torch.from_numpy(np.stack([x[i] for x in kv])).cuda()
                            for i in range(2)))
    bm = pkv.BlockManager(nb, bs, free_order=sched.free_order)
    ids = [bm.add_sequence() for _ in range(B)]
    for s in range(B):
        bm.prepare_write(ids[s], 0, int(sched.prompt_lens[s]))
    tables = torch.from_numpy(bm.tables(ids, W)).cuda()
    cu = torch.from_numpy(
        np.concatenate([[0], np.cumsum(sched.prompt_lens)]).astype(np.int32)).cuda()
    zero = torch.zeros(B, dtype=torch.int32, device="cuda")
    for l in range(L):
        k, v = replay_step_values(sched, -1, l, list(range(B)), "kv")
        pkv.kv_append(kc[l], vc[l], torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                      tables, zero, cu)
    torch.cuda.synchronize()
    total_bytes, total_tokens, calls = 0, 0, 0
    out = torch.empty((B, hq, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(pkv.decode_workspace_bytes(B, hq, d, 320, 0), dtype=torch.uint8,
                     device="cuda")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    seq_ids = np.asarray(ids, np.int32)
    prompt = np.asarray(sched.prompt_lens, np.int32)
    gen = np.asarray(sched.gen_lens, np.int32)
    ones = np.ones(B, np.int32)
    # a step's tables [n, W], start [n], ctx [n] and cu [n + 1] go up in one copy, from two
    # pinned host buffers in turn into two device buffers in turn.  The copy is queued
    # behind the previous step's launches instead of waiting for them (a copy from pageable
    # memory would), so the host prepares step t + 1 while the GPU runs step t.  A host
    # buffer is rewritten only after the copy that last read it has run (its event).
    m_max = B * W + 3 * B + 1
    stage = [torch.empty(m_max, dtype=torch.int32).pin_memory() for _ in range(2)]
    stage_np = [x.numpy() for x in stage]
    stage_dev = [torch.empty(m_max, dtype=torch.int32, device="cuda") for _ in range(2)]
    stage_ev = [torch.cuda.Event() for _ in range(2)]
    t0 = time.perf_counter()
    ev0.record()
    for t in range(steps):
        active = plan[t]
        n = len(active)
        act = np.asarray(active, np.intp)
        pos = prompt[act] + t
        i = t & 1
        stage_ev[i].synchronize()
        host = stage_np[i]
        # every sequence's next slot made writable and the tables written in one call
        bm.prepare_step(seq_ids[act], pos, ones[:n], W, tables_out=host[:n * W].reshape(n, W))
        host[n * W:n * W + n] = pos
        host[n * W + n:n * W + 2 * n] = pos + 1
        host[n * W + 2 * n:n * W + 3 * n + 1] = np.arange(n + 1, dtype=np.int32)
        m = n * W + 3 * n + 1
        dev_all = stage_dev[i][:m]
        dev_all.copy_(stage[i][:m], non_blocking=True)
        stage_ev[i].record()
        d_tables = dev_all[:n * W].view(n, W)
        d_start = dev_all[n * W:n * W + n]
        d_ctx = dev_all[n * W + n:n * W + 2 * n]
        d_cu = dev_all[n * W + 2 * n:]
        max_ctx = int(pos.max()) + 1
        # one work plan for the step, then one append + decode launch per layer: two
        # library calls, the step's tensors checked once
        k_new, v_new = kv_all[t]
        pkv.append_paged_decode_layers(q_all[t], kc, vc, k_new, v_new, d_tables, d_start, d_cu,
                                       d_ctx, max_ctx, ws, partition_size=0, out=out[:n])
        calls += L
        ctxs = (pos + 1).astype(np.int64)
        total_tokens += L * int(ctxs.sum())
        total_bytes += L * (int(ctxs.sum()) * 2 * hkv * d * 4 + n * (hq * d * 4 * 2 + 4) +
                            int(((ctxs + 15) // 16).sum()) * 4 + n * (2 * 2 * hkv * d * 4 + 12))
        for s in act[gen[act] == t + 1]:
            bm.free_sequence(ids[s])
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_s = ev0.elapsed_time(ev1) / 1e3
    flags = pkv.device_error()
    if flags:
        raise RuntimeError(f"device error: {pkv.describe_device_error(flags)}")
    return {
        "metric": "paged decode attention achieved HBM GB/s (% of peak) + seq-tokens/s at 1 GPU",
        "value": round(total_bytes / wall / 1e9, 3),
        "unit": "GB/s",
        "n_gpus": 1, "steps": steps, "warmup": 0,
        "ms_per_step": round(wall / steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "gpt2_replay", "seed": args.seed, "batch": B, "layers": L,
                   "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": d, "block_size": bs,
                   "num_blocks": nb, "steps": steps,
                   "step": "host block manager + table upload + work plan, then per layer one "
                           "append + decode launch, every layer issued by one library call"},
        "pct_of_hbm_peak": round(100 * total_bytes / wall / 1e9 / HBM_PEAK_GBPS, 3),
        "seq_tokens_per_s": round(total_tokens / wall, 1),
        "gpu_event_seconds": round(gpu_s, 5),
        "wall_seconds": round(wall, 5),
        "decode_calls": calls,
        "algorithmic_bytes": total_bytes,
        "note": "launch- and host-bound: each layer call moves about 6 MB",
    }


CROSSOVER_BATCHES = (1, 4, 16, 64, 256)
CROSSOVER_CONTEXTS = (512, 2048, 8192, 32768)
CROSSOVER_PARTS = (0, 256, 512, 1024, 2048, 4096, 8192)
CROSSOVER_MAX_TOKENS = 1 << 21  # 8.6 GB of bf16 K+V at 8 KV heads x 128 dims


def run_crossover(args, np, torch, pkv):
    """Decode-call time (plan + first pass + combine when needed) for uniform-length bf16
    workloads (32 query / 8 KV heads, head_dim 128, blocks randomly permuted), over batch x
    context x partition size (0 = one unit per sequence and KV head)."""
    hq, hkv, d = 32, 8, 128
    rows = []
    gen = torch.Generator(device="cuda")
    gen.manual_seed(args.seed)
    for B in CROSSOVER_BATCHES:
        for n in CROSSOVER_CONTEXTS:
            if B * n > CROSSOVER_MAX_TOKENS:
                continue
            nb = B * n // 16
            k = torch.randn((nb + 1, hkv, 16, d), generator=gen, device="cuda",
                            dtype=torch.bfloat16)
            v = torch.randn((nb + 1, hkv, 16, d), generator=gen, device="cuda",
                            dtype=torch.bfloat16)
            tables = torch.randperm(nb, generator=gen, device="cuda").to(torch.int32)
            tables = tables.view(B, n // 16).contiguous()
            ctx = torch.full((B,), n, dtype=torch.int32, device="cuda")
            q = torch.randn((B, hq, d), generator=gen, device="cuda", dtype=torch.bfloat16)
            out = torch.empty((B, hq, d), dtype=torch.float32, device="cuda")
            lse = torch.empty((B, hq), dtype=torch.float32, device="cuda")
            byt = B * n * 2 * hkv * d * 2
            line = {"batch": B, "context": n, "kv_bytes": byt, "us": {}}
            for P in CROSSOVER_PARTS:
                if P >= n:  # one partition: the same work as P = 0
                    continue
                ws = torch.empty(max(1, pkv.decode_workspace_bytes(B, hq, d, n, P)),
                                 dtype=torch.uint8, device="cuda")

                def call():
                    pkv.paged_decode(q, k, v, tables, ctx, n, partition_size=P, out=out,
                                     lse=lse, workspace=ws)

                for _ in range(3):
                    call()
                s_ev = torch.cuda.Event(enable_timing=True)
                e_ev = torch.cuda.Event(enable_timing=True)
                reps = 20
                s_ev.record()
                for _ in range(reps):
                    call()
                e_ev.record()
                torch.cuda.synchronize()
                line["us"][P] = round(s_ev.elapsed_time(e_ev) * 1e3 / reps, 2)
            best = min(line["us"], key=line["us"].get)
            line["best_partition"] = best
            line["best_gbps"] = round(byt / line["us"][best] / 1e3, 1)
            rows.append(line)
            print(f"[crossover] batch {B:4d} ctx {n:6d}: " +
                  " ".join(f"P{P}={t:.1f}" for P, t in line["us"].items()) +
                  f"  best P{best} ({line['best_gbps']} GB/s)", file=sys.stderr, flush=True)
            del k, v, tables, ctx, q, out, lse
    flags = pkv.device_error()
    if flags:
        raise RuntimeError(f"device error: {pkv.describe_device_error(flags)}")
    return {"metric": "paged decode call time by batch x context x partition size (us)",
            "unit": "us", "n_gpus": 1, "higher_is_better": False, "dtype": "bf16",
            "data": "synthetic", "config": {"workload": "crossover sweep", "num_q_heads": hq,
                                            "num_kv_heads": hkv, "head_dim": d,
                                            "block_size": 16, "lengths": "uniform"},
            "rows": rows}


def main():
    args = parse_args()
    # No cyclic garbage collection in this process: a full collection traverses every
    # tensor and array made while building the inputs (about 40 ms on the replay's), and
    # would land inside one timed step at random.  Reference counting frees the rest.
    gc.disable()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this decode path has no "
              "multi-GPU mode; sharding by sequence or KV head needs no collective.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import paged_kv_cache_200_amd as pkv
    from workloads import config_case, decode_step_inputs, fork_groups

    if args.crossover:
        print(json.dumps(run_crossover(args, np, torch, pkv)), flush=True)
        return
    if args.workload == "gpt2_replay":
        print(json.dumps(run_replay(args, np, torch, pkv)), flush=True)
        return
    if args.workload == "chunked_prefill":
        print(json.dumps(run_prefill(args, np, torch, pkv)), flush=True)
        return

    print(f"[bench] building inputs: {args.workload} seed {args.seed}", file=sys.stderr, flush=True)
    case = config_case(args.workload, args.seed)
    shared_path = case.fork_parent is not None and not args.no_shared_prefix
    mfma_plain = args.decode_path == "mfma" and case.fork_parent is None
    if mfma_plain:
        if case.kv_dtype != "bf16":
            print("--decode-path mfma needs a bf16 workload", file=sys.stderr)
            sys.exit(2)
        shared_path = True
    if args.partition_size is not None:
        P = args.partition_size
    elif "partition_size" in case.extra:
        P = case.extra["partition_size"]  # the workload states its own
    elif shared_path and not mfma_plain:
        P = 1024
    else:
        # the library's rule, from the sizes the host knows
        P = pkv.decode_partition_size(case.batch, case.num_kv_heads, case.head_dim,
                                      int(case.context_lens.max()),
                                      int(case.context_lens.sum()))
    if args.workload == "tiny":
        P = 0
    B, hq, hkv, d = case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim
    layers = case.layers

    def to_dev(x):
        if x.dtype == np.uint16:
            x = x.view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()

    # every layer's q and caches stacked on a leading layer dimension; qs[l] etc. are views
    q_st, kc_st, vc_st = (to_dev(x[:layers]) for x in (case.q, case.k_pool, case.v_pool))
    qs, kcs, vcs = list(q_st), list(kc_st), list(vc_st)
    q, kc, vc = qs[0], kcs[0], vcs[0]
    tables = to_dev(case.block_tables)
    ctx = to_dev(case.context_lens)
    max_ctx = int(case.context_lens.max())
    # the token appended this step sits at position ctx - 1 (it attends to itself); fork
    # members without a private block append nothing (copy-on-write)
    si = decode_step_inputs(case, args.seed)
    start, cu = to_dev(si.start_pos), to_dev(si.cu_new)
    total_new = int(si.cu_new[-1])
    k_new, v_new = to_dev(si.k_new), to_dev(si.v_new)
    out = torch.empty((B, hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, hq), dtype=torch.float32, device="cuda")
    if mfma_plain:
        # every sequence its own group, nothing shared: the matrix-core tile on plain decode
        gs_np, gb_np = np.arange(B + 1, dtype=np.int32), np.zeros(B, np.int32)
        gstarts, gblocks, max_shared = to_dev(gs_np), to_dev(gb_np), 0
        ws_bytes = pkv.shared_prefix_workspace_bytes(B, hq, d, max_ctx, P)
    elif shared_path:
        gs_np, gb_np = fork_groups(case)
        gstarts, gblocks, max_shared = to_dev(gs_np), to_dev(gb_np), int(gb_np.max())
        ws_bytes = pkv.shared_prefix_workspace_bytes(B, hq, d, max_ctx, P)
    else:
        ws_bytes = pkv.decode_workspace_bytes(B, hq, d, max_ctx, P)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    scale = float(case.scale)

    def shared_decode(l):
        pkv.paged_decode_shared_prefix(qs[l], kcs[l], vcs[l], tables, ctx, gstarts, gblocks,
                                       max_shared, max_ctx, scale=scale, partition_size=P,
                                       out=out, lse=lse, workspace=ws)

    in_pass = not shared_path and (args.append_in_pass == "yes" or
                                   (args.append_in_pass == "auto" and layers > 1))
    if in_pass:
        step_plan = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
        # each layer appends this step's token rows to its own cache: the rows stacked
        # per layer for the one-call form
        kn_st, vn_st = (x.expand(layers, *x.shape).contiguous() for x in (k_new, v_new))

    def step():
        if in_pass:
            # lengths advance once per step, so one plan serves every layer: the step-wide
            # tensors are checked and planned once, then one library call launches every
            # layer's append + decode
            ds = pkv.DecodeStep(qs[0], kcs[0], vcs[0], k_new, v_new, tables, start, cu, ctx,
                                max_ctx, scale=scale, partition_size=P, out=out, lse=lse,
                                workspace=step_plan)
            ds.layers(q_st, kc_st, vc_st, kn_st, vn_st)
            return
        for l in range(layers):
            if shared_path:
                # fork groups: append and work plan in one launch, then one decode launch
                # that streams each group's shared blocks once for all members
                pkv.append_paged_decode_shared_prefix(
                    qs[l], kcs[l], vcs[l], k_new, v_new, tables, start, cu, ctx, gstarts,
                    gblocks, max_shared, max_ctx, scale=scale, partition_size=P, out=out,
                    lse=lse, workspace=ws)
            else:
                # kv_append + paged_decode in one library call (append and work plan
                # share a launch)
                pkv.append_paged_decode(qs[l], kcs[l], vcs[l], k_new, v_new, tables, start,
                                        cu, ctx, max_ctx, scale=scale, partition_size=P,
                                        out=out, lse=lse, workspace=ws)

    if args.calibrate_copy > 0:
        n = args.calibrate_copy << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copies: 3 x {n} bytes read + written", file=sys.stderr,
              flush=True)
        del src, dst

    run = step
    if args.graph:
        # the whole step (every layer's launches) as one HIP graph: same kernels and
        # inputs, no per-call host work between them
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        run = graph.replay

    print("[bench] warmup", file=sys.stderr, flush=True)
    settle(run, torch, args.settle_seconds)
    for _ in range(args.warmup):
        run()
    # (no device-error read here: it waits on the GPU and would leave it idle, clocks
    # falling, just before the timed steps; the error word is read after them)

    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    if args.cold:
        # every step on its own, after a 1 GiB write that evicts L2 and Infinity Cache
        # The sweep reads: a written sweep would leave the Infinity Cache full of dirty
        # lines, and a step whose loads allocate there would pay their write-back.  (No host
        # synchronisation between steps: while the GPU sweeps, the host enqueues the step.)
        scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        marks = []
        for i in range(args.steps):
            scratch.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run()
            e1.record(stream)
            marks.append((e0, e1))
        torch.cuda.synchronize()
        per_step = np.array([e0.elapsed_time(e1) for e0, e1 in marks])
        ms_per_step = float(np.mean(per_step))
        wall = time.perf_counter() - t0
        del scratch
    else:
        # the K steps between two events only: an event recorded after every step added
        # 2.3-3.5 us to each ~227 us step of the headline workload
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_per_step = e0.elapsed_time(e1) / args.steps
        wall = time.perf_counter() - t0
        # the spread of single steps, from a second run of K steps with an event after each
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        evs[0].record(stream)
        for i in range(args.steps):
            run()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        per_step = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    flags = pkv.device_error()
    if flags:
        raise RuntimeError(f"device error: {pkv.describe_device_error(flags)}")
    print(f"[bench] {args.steps} steps{' (cold)' if args.cold else ''}: "
          f"{ms_per_step * 1e3:.1f} us/step (wall {wall:.3f} s)", file=sys.stderr, flush=True)

    # the first pass alone, as the step launches it: the planned decode on a plan computed
    # beforehand is that single launch when split sequences are merged inside it; past
    # the library's in-pass limit the combine is a launch of its own, and the first pass
    # is timed without it
    plan_ws = pkv.decode_plan(ctx, tables, hq, d, max_ctx, P)
    np_max = max(1, -(-max_ctx // P)) if P > 0 else 1
    timed_kernel = ("decode_mfma_kernel"
                    if pkv.decode_engine(case.kv_dtype, d, hq, hkv) == "matrix"
                    else "decode_pass1_kernel")
    if shared_path:
        # no single dominant kernel: the whole decode call (plan, shared-prefix pass, first
        # pass over the private ranges, combine) against the unique bytes
        timed_kernel = "paged_decode_shared_prefix call"

        def pass1():
            shared_decode(0)
    elif np_max > pkv.IN_PASS_MERGE_MAX_PARTITIONS:
        part_out = torch.empty((B, hq, np_max, d), dtype=torch.float32, device="cuda")
        part_lse = torch.empty((B, hq, np_max), dtype=torch.float32, device="cuda")

        def pass1():
            pkv.paged_decode_partials(q, kc, vc, tables, ctx, max_ctx, P, scale=scale,
                                      part_out=part_out, part_lse=part_lse,
                                      plan_workspace=plan_ws)
    else:
        def pass1():
            pkv.paged_decode_planned(q, kc, vc, tables, ctx, max_ctx, plan_ws, scale=scale,
                                     partition_size=P, out=out, lse=lse)

    # the launches ahead of the timed ones are not waited for (the GPU stays busy up to
    # the first timed launch); the cold timing waits before each of its sweeps anyway
    for _ in range(5):
        pass1()
    if args.cold:
        scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        marks = []
        for i in range(args.kernel_reps):
            scratch.sum()
            ks, ke = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ks.record(stream)
            pass1()
            ke.record(stream)
            marks.append((ks, ke))
        torch.cuda.synchronize()
        pass1_s = float(np.mean([ks.elapsed_time(ke) for ks, ke in marks])) / 1e3
        del scratch
    else:
        ks, ke = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ks.record(stream)
        for _ in range(args.kernel_reps):
            pass1()
        ke.record(stream)
        torch.cuda.synchronize()
        pass1_s = ks.elapsed_time(ke) / 1e3 / args.kernel_reps
    flags = pkv.device_error()
    if flags:
        raise RuntimeError(f"device error: {pkv.describe_device_error(flags)}")

    decode_bytes, append_bytes = algorithmic_bytes(case, total_new)
    # shared (copy-on-write) blocks need to come from HBM once per call
    logical_tokens = int(case.context_lens.sum())
    unique_tokens = unique_kv_tokens(case) if case.shared_blocks else logical_tokens
    kv_tok = 2 * hkv * d * case.elem_bytes
    p1_bytes = decode_bytes - (logical_tokens - unique_tokens) * kv_tok
    step_s = ms_per_step / 1e3
    step_bytes = layers * (p1_bytes + append_bytes)
    value = step_bytes / step_s / 1e9
    achieved = p1_bytes / pass1_s / 1e9
    traffic = traffic_from_profile(args.workload, P, args.seed)

    # Back to back, a step whose bytes fit the Infinity Cache finds most of them there:
    # then every step is also timed after a 1 GiB read that evicts them (outside its events).
    cold_ms = None
    if not args.cold and step_bytes < INFINITY_CACHE_BYTES:
        scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        marks = []
        for _ in range(args.steps):
            scratch.sum()
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record(stream)
            run()
            c1.record(stream)
            marks.append((c0, c1))
        torch.cuda.synchronize()
        cold_ms = float(np.mean([c0.elapsed_time(c1) for c0, c1 in marks]))
        del scratch

    probe = None if args.no_copy_probe else copy_probe(torch)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(case, p1_bytes, args.cpu_seconds)

    sum_ctx = layers * logical_tokens
    line = {
        "metric": "paged decode attention achieved HBM GB/s (% of peak) + seq-tokens/s at 1 GPU",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": args.settle_seconds,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.kv_dtype,
        "data": "synthetic",
        "config": {
            "workload": case.name,
            "seed": args.seed,
            "batch": B,
            "num_q_heads": hq,
            "num_kv_heads": hkv,
            "head_dim": d,
            "block_size": 16,
            "sum_context_tokens": sum_ctx,
            "max_context_len": max_ctx,
            "num_blocks": case.num_blocks,
            "layers": layers,
            "partition_size": P,
            "step": ("append + work plan (one launch), shared-prefix and private ranges (one "
                     "launch), LSE combine"
                     if shared_path else
                     "work plan (one launch per step), then per layer one launch that appends "
                     "1 token/seq and runs the split-KV first pass with the LSE merge"
                     + ("" if np_max <= pkv.IN_PASS_MERGE_MAX_PARTITIONS
                        else ", then the LSE combine (one launch)")
                     if in_pass else
                     "append 1 token/seq + work plan (one launch), split-KV first pass with "
                     "the LSE merge of split sequences in the same launch"
                     if np_max <= pkv.IN_PASS_MERGE_MAX_PARTITIONS else
                     "append 1 token/seq + work plan (one launch), split-KV first pass, "
                     "LSE combine (one launch)"),
            "appended_tokens_per_layer": total_new,
            "launch": "hip graph of the whole step" if args.graph else "eager",
            "decode_path": ("matrix-core tile, groups of one" if mfma_plain else
                            "shared-prefix" if shared_path else
                            "matrix-core first pass" if timed_kernel == "decode_mfma_kernel"
                            else "VALU first pass"),
            "caches": ("cold: 1 GiB read before every step" if args.cold
                       else "warm: steps back to back"),
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "seq_tokens_per_s": round(sum_ctx / step_s, 1),
        "step_ms_p10_p50_p90": [round(float(np.percentile(per_step, p)), 5) for p in (10, 50, 90)],
        "cold_ms_per_step": None if cold_ms is None else round(cold_ms, 5),
        "cold_gbps": None if cold_ms is None else round(step_bytes / (cold_ms / 1e3) / 1e9, 2),
        "algorithmic_bytes_per_step": step_bytes,
        "logical_kv_bytes_per_layer": logical_tokens * kv_tok,
        "unique_kv_bytes_per_layer": unique_tokens * kv_tok,
        "roofline": {
            "kernel": timed_kernel,
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": p1_bytes,
            "avg_launch_us": round(pass1_s * 1e6, 2),
        },
        "copy_probe_gbps": None if probe is None else round(probe, 1),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
