"""Block-table and append indexing, exact against the oracle on every shipped path.

Each case is a one-hot gather probe (tests/probe_util.py): every query row's exact result
is one stored V row, which the float64 oracle also returns once rounded to float32
(tests/test_probe_pins.py); results must equal it value for value (a zero's sign aside).
Over the rounds of a case every (KV head, dimension) of every sequence is probed, so the
hot keys cover every block position of sequences up to Hkv * D blocks per phase, and
phases shift the window for longer ones.  Paths:
  decode    pkv_paged_decode                      (plan + first pass; combine past 8 parts)
  append    pkv_append_paged_decode               (append + plan in one launch, first pass)
  in_pass   pkv_decode_plan + pkv_append_paged_decode_planned (the first pass appends)
  partials  pkv_paged_decode_partials + pkv_lse_combine
  shared1   pkv_paged_decode_shared_prefix, every sequence a group of one (bf16: the
            matrix-core tile on plain decode)
plus the shared-prefix decode of fork groups, DecodeStep over several layers, the paged
prefill (bf16 matrix cores and fp32 VALU) and the exact calls bench.py times.  For the
append paths the newest token's slot holds NaN before the call and the probe's key for
it arrives in k_new, so a misplaced append is visible twice: in the pool, compared
bytewise with the oracle's kv_append, and in the attention result."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.paged_attention as pa
from gpu_util import assert_no_device_error, dev, say
from libpkv_util import ensure_built
from probe_util import (decode_probe, decode_round_q, decode_rounds, fork_probe, hot_rows,
                        prefill_expected, prefill_probe, round_expected, v_rows)
from workloads import (build_case, chunked_prefill_case, config_case, decode_step_inputs,
                       fork_case, fork_groups)

pytestmark = pytest.mark.gpu

F32_QNAN = np.uint32(0x7FC00000)
BF16_QNAN = np.uint16(0x7FC0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ensure_built()


def _ops():
    from paged_kv_cache_200_amd import ops
    return ops


def _nan(kv_dtype):
    return F32_QNAN if kv_dtype == "f32" else BF16_QNAN


def _bits(pool, kv_dtype):
    return pool.view(np.uint32) if kv_dtype == "f32" else pool


def _same(got: torch.Tensor, want: np.ndarray, what: str):
    """Every element equal as a float32 value (NaN never equal).  A stored -0.0 may come
    back as +0.0: the kernels' weighted sums start from +0, and +0 + -0 is +0; the float64
    oracle's sign for such an element is that of its ~1e-70 remainder, so no sign of zero
    is the reference one."""
    g = got.cpu().numpy()
    if not np.array_equal(g, want):
        bad = np.argwhere(np.any(g != want, axis=-1))
        raise AssertionError(f"{what}: {len(bad)} rows differ from the hot V rows, "
                             f"first {bad[:5].tolist()}")


class StepProbe:
    """One layer's probe pools, before and after the step's append of each sequence's
    newest token (appending: which sequences append)."""

    def __init__(self, case, layer=0, appending=None):
        self.case = case
        kvd = case.kv_dtype
        B = case.batch
        self.post_k, self.post_v = case.k_pool[layer], case.v_pool[layer]
        lens = case.context_lens
        app = (lens > 0) if appending is None else (np.asarray(appending) & (lens > 0))
        self.start = (lens - 1).clip(min=0).astype(np.int32)
        self.cu = np.concatenate([[0], np.cumsum(app)]).astype(np.int32)
        sl = [(int(case.block_tables[s, (lens[s] - 1) // 16]), int((lens[s] - 1) % 16))
              for s in range(B) if app[s]]
        blk = np.array([b for b, _ in sl], np.int64)
        slot = np.array([t for _, t in sl], np.int64)
        D = case.head_dim
        shape = (len(sl), case.num_kv_heads, D)
        self.k_new = self.post_k[blk, :, slot].reshape(shape).copy()
        self.v_new = self.post_v[blk, :, slot].reshape(shape).copy()
        self.pre_k, self.pre_v = self.post_k.copy(), self.post_v.copy()
        for pool in (self.pre_k, self.pre_v):
            _bits(pool, kvd)[blk, :, slot] = _nan(kvd)
        # the oracle's append of the new rows into the pre-step pools is the post pools
        wk, wv = pa.kv_append(self.pre_k, self.pre_v, self.k_new, self.v_new,
                              case.block_tables, self.start, self.cu)
        assert wk.tobytes() == self.post_k.tobytes() and wv.tobytes() == self.post_v.tobytes()


class DevProbe:
    """Device tensors of a StepProbe and the decode paths run on them."""

    def __init__(self, sp: StepProbe, paths):
        c = sp.case
        self.sp = sp
        self.tables, self.ctx = dev(c.block_tables), dev(c.context_lens)
        self.max_ctx = int(c.context_lens.max()) if c.batch else 0
        self.start, self.cu = dev(sp.start), dev(sp.cu)
        self.k_new, self.v_new = dev(sp.k_new), dev(sp.v_new)
        # each appending path gets pools of its own, holding NaN in the appended slots
        self.pre = {p: (dev(sp.pre_k), dev(sp.pre_v)) for p in paths if p in ("append", "in_pass")}
        if any(p not in self.pre for p in paths):
            self.k, self.v = dev(sp.post_k), dev(sp.post_v)
        B = c.batch
        self.gstarts = dev(np.arange(B + 1, dtype=np.int32))
        self.gblocks = dev(np.zeros(B, np.int32))
        self.checked = set()

    def run(self, path, q, P):
        ops = _ops()
        c = self.sp.case
        if path == "decode":
            o, _ = ops.paged_decode(q, self.k, self.v, self.tables, self.ctx, self.max_ctx,
                                    scale=1.0, partition_size=P)
        elif path == "append":
            k, v = self.pre[path]
            o, _ = ops.append_paged_decode(q, k, v, self.k_new, self.v_new,
                                           self.tables, self.start, self.cu, self.ctx,
                                           self.max_ctx, scale=1.0, partition_size=P)
        elif path == "in_pass":
            ws = ops.decode_plan(self.ctx, self.tables, c.num_q_heads, c.head_dim,
                                 self.max_ctx, P)
            k, v = self.pre[path]
            o, _ = ops.append_paged_decode_planned(q, k, v, self.k_new,
                                                   self.v_new, self.tables, self.start,
                                                   self.cu, self.ctx, self.max_ctx, ws,
                                                   scale=1.0, partition_size=P)
        elif path == "partials":
            po, pl = ops.paged_decode_partials(q, self.k, self.v, self.tables, self.ctx,
                                               self.max_ctx, P, scale=1.0)
            o, _ = ops.lse_combine(po, pl, self.ctx, P)
        elif path == "shared1":
            o, _ = ops.paged_decode_shared_prefix(q, self.k, self.v, self.tables, self.ctx,
                                                  self.gstarts, self.gblocks, 0, self.max_ctx,
                                                  scale=1.0, partition_size=P)
        else:
            raise ValueError(path)
        torch.cuda.synchronize()
        if path in self.pre and path not in self.checked:
            k, v = self.pre[path]
            assert k.cpu().numpy().tobytes() == self.sp.post_k.tobytes(), \
                f"{path}: K pool after the append differs from the oracle's kv_append"
            assert v.cpu().numpy().tobytes() == self.sp.post_v.tobytes(), \
                f"{path}: V pool after the append differs from the oracle's kv_append"
            self.checked.add(path)
        return o


def _phases(case):
    most = max([-(-int(n) // 16) for n in case.context_lens] + [1])
    return -(-most // (case.num_kv_heads * case.head_dim))


def _probe_decode(case, paths, P, seed, what):
    """Every phase and round of a decode probe through each path."""
    hq, hkv, d, kvd = case.num_q_heads, case.num_kv_heads, case.head_dim, case.kv_dtype
    case.scale = np.float32(1.0)
    for phase in range(_phases(case)):
        hot = decode_probe(case, 0, phase, seed=seed + phase)
        rows = hot_rows(case.v_pool[0], case.block_tables, case.context_lens, hot, kvd)
        dp = DevProbe(StepProbe(case), paths)
        for r in range(decode_rounds(hq, hkv, d)):
            qh, dims = decode_round_q(case.batch, hq, hkv, d, r, kvd)
            want = round_expected(rows, dims, hq)
            q = dev(qh)
            for path in paths:
                _same(dp.run(path, q, P), want, f"{what} {path} P{P} phase {phase} round {r}")
        say(f"  {what} P{P} {paths}: {_phases(case)} phase(s) x "
            f"{decode_rounds(hq, hkv, d)} rounds bit-exact")
    assert_no_device_error()


SHAPES = [("bf16", 32, 8, 128), ("bf16", 14, 2, 64), ("f32", 12, 12, 64), ("f32", 8, 2, 128)]
# past the 64-block id window of a wave (4096 tokens with four waves), odd and even
# windows, partial last blocks, and short ones
LENS = [1, 17, 300, 4097, 8193, 9000]


@pytest.mark.parametrize("kv_dtype,hq,hkv,d", SHAPES)
@pytest.mark.parametrize("P", [0, 512, 4096])
def test_probe_decode_paths(kv_dtype, hq, hkv, d, P):
    say(f"probe decode {kv_dtype} {hq}/{hkv}x{d} P{P}")
    case = build_case("probe", LENS, hq, hkv, d, kv_dtype, seed=hq + d + P)
    paths = ["decode", "append", "in_pass", "shared1"] + (["partials"] if P else [])
    _probe_decode(case, paths, P, seed=P + d, what=f"{kv_dtype} {hq}/{hkv}x{d}")


@pytest.mark.parametrize("P", [512, 4096, 0])
def test_probe_long_context(P):
    """4 x 32768 tokens: 2048 blocks per sequence, two phases."""
    say(f"probe long_context P{P}")
    case = config_case("long_context", 0)
    paths = ["decode", "append", "in_pass"] + (["partials", "shared1"] if P == 512 else [])
    _probe_decode(case, paths, P, seed=11, what="long_context")


@pytest.mark.parametrize("seed,rule", [(0, True), (1, True), (2, True), (0, False)])
def test_probe_high_concurrency_as_benched(seed, rule):
    """The benched call (append + decode at the library's partition-size rule, which is
    no split here) on the full 256-sequence workload of each seed; seed 0 also through the
    in-pass append that DecodeStep uses, and at partition 4096 (split, merged in the
    pass)."""
    from paged_kv_cache_200_amd import ops
    case = config_case("high_concurrency", seed)
    P = (ops.decode_partition_size(case.batch, 8, 128, int(case.context_lens.max()),
                                   int(case.context_lens.sum())) if rule else 4096)
    say(f"probe high_concurrency seed {seed} P{P}")
    paths = ["append", "in_pass"] if seed == 0 else ["append"]
    _probe_decode(case, paths, P, seed=seed, what=f"high_concurrency s{seed}")


@pytest.mark.parametrize("P", [512, 0])
def test_probe_decode_step_layers(P):
    """DecodeStep over three Qwen-shaped layers (one plan, one launch per layer that
    appends and attends), each layer its own probe."""
    say(f"probe DecodeStep qwen_gqa x3 P{P}")
    ops = _ops()
    case = config_case("qwen_gqa", 1, layers=3)
    case.scale = np.float32(1.0)
    hq, hkv, d = case.num_q_heads, case.num_kv_heads, case.head_dim
    for phase in range(_phases(case)):
        sps, rows = [], []
        for layer in range(3):
            hot = decode_probe(case, layer, phase, seed=100 * layer + phase)
            rows.append(hot_rows(case.v_pool[layer], case.block_tables, case.context_lens, hot,
                                 "bf16"))
            sps.append(StepProbe(case, layer))
        tables, ctx = dev(case.block_tables), dev(case.context_lens)
        start, cu = dev(sps[0].start), dev(sps[0].cu)
        ks = [dev(sp.pre_k) for sp in sps]
        vs = [dev(sp.pre_v) for sp in sps]
        kn = [dev(sp.k_new) for sp in sps]
        vn = [dev(sp.v_new) for sp in sps]
        max_ctx = int(case.context_lens.max())
        for r in range(decode_rounds(hq, hkv, d)):
            qh, dims = decode_round_q(case.batch, hq, hkv, d, r, "bf16")
            q = dev(qh)
            step = ops.DecodeStep(q, ks[0], vs[0], kn[0], vn[0], tables, start, cu, ctx,
                                  max_ctx, scale=1.0, partition_size=P)
            for layer in range(3):
                o, _ = step.layer(q, ks[layer], vs[layer], kn[layer], vn[layer], out=torch.empty_like(step.out))
                torch.cuda.synchronize()
                _same(o, round_expected(rows[layer], dims, hq),
                      f"DecodeStep layer {layer} P{P} phase {phase} round {r}")
        for layer in range(3):
            assert ks[layer].cpu().numpy().tobytes() == sps[layer].post_k.tobytes()
            assert vs[layer].cpu().numpy().tobytes() == sps[layer].post_v.tobytes()
    assert_no_device_error()


def _fork_probe_run(case, P, append, what):
    ops = _ops()
    kvd = case.kv_dtype
    hq, hkv, d = case.num_q_heads, case.num_kv_heads, case.head_dim
    case.scale = np.float32(1.0)
    gs, gb = fork_groups(case)
    hot = fork_probe(case, gs, gb, 0, seed=5)
    rows = hot_rows(case.v_pool[0], case.block_tables, case.context_lens, hot, kvd)
    si = decode_step_inputs(case, 0)
    appending = np.diff(si.cu_new) > 0
    sp = StepProbe(case, 0, appending if append else np.zeros(case.batch, bool))
    tables, ctx = dev(case.block_tables), dev(case.context_lens)
    gsd, gbd = dev(gs), dev(gb)
    k, v = dev(sp.pre_k), dev(sp.pre_v)
    max_ctx = int(case.context_lens.max())
    for r in range(decode_rounds(hq, hkv, d)):
        qh, dims = decode_round_q(case.batch, hq, hkv, d, r, kvd)
        q = dev(qh)
        if append:
            o, _ = ops.append_paged_decode_shared_prefix(
                q, k, v, dev(sp.k_new), dev(sp.v_new), tables, dev(sp.start), dev(sp.cu), ctx,
                gsd, gbd, int(gb.max()), max_ctx, scale=1.0, partition_size=P)
        else:
            o, _ = ops.paged_decode_shared_prefix(q, k, v, tables, ctx, gsd, gbd, int(gb.max()),
                                                  max_ctx, scale=1.0, partition_size=P)
        torch.cuda.synchronize()
        _same(o, round_expected(rows, dims, hq), f"{what} P{P} round {r}")
    assert k.cpu().numpy().tobytes() == sp.post_k.tobytes(), "K pool after the step"
    assert v.cpu().numpy().tobytes() == sp.post_v.tobytes(), "V pool after the step"
    say(f"  {what} P{P}: {decode_rounds(hq, hkv, d)} rounds bit-exact")
    assert_no_device_error()


@pytest.mark.parametrize("P,append", [(1024, True), (512, False), (0, False), (4096, True)])
def test_probe_prefix_fork_as_benched(P, append):
    """The 64-fork workload (16 parents x 4, 2048-token shared prefixes) through the
    shared-prefix path; P = 1024 with the append is the benched call."""
    say(f"probe prefix_fork P{P} append={append}")
    _fork_probe_run(config_case("prefix_fork", 0), P, append, "prefix_fork")


@pytest.mark.parametrize("kv_dtype,hq,hkv,d", [("bf16", 32, 8, 128), ("bf16", 14, 2, 64),
                                               ("f32", 12, 12, 64), ("bf16", 8, 8, 128)])
@pytest.mark.parametrize("P", [0, 256])
def test_probe_fork_groups(kv_dtype, hq, hkv, d, P):
    """Groups of 1 to 8 members, aligned and unaligned prefixes, members without private
    tokens, prefixes past the 4096-token id window."""
    prefixes = [20, 4112, 304, 33, 1024]
    forks = [3, 4, 8, 1, 2]
    priv = [[0, 0, 0], [0, 100, 17, 4000], [5, 0, 1, 2, 3, 200, 16, 31], [0], [700, 0]]
    say(f"probe fork groups {kv_dtype} {hq}/{hkv}x{d} P{P}")
    case = fork_case("forkprobe", prefixes, forks, priv, hq, hkv, d, kv_dtype, seed=hq + P)
    _fork_probe_run(case, P, False, f"forks {kv_dtype} {hq}/{hkv}x{d}")


def _prefill_probe_run(case, k_new, v_new, cu, start, what, seed=0):
    """kv_append of the chunks, then paged_prefill, on a prefill probe."""
    ops = _ops()
    kvd = case.kv_dtype
    case.scale = np.float32(1.0)
    q, hot = prefill_probe(case, k_new, cu, start, 0, seed=seed)
    kp, vp = pa.kv_append(case.k_pool[0], case.v_pool[0], k_new, v_new, case.block_tables,
                          start, cu)
    vseq = v_rows(vp, case.block_tables, case.context_lens, kvd)
    want = prefill_expected(vseq, hot, cu, case.num_q_heads, case.num_kv_heads)
    k, v = dev(case.k_pool[0]), dev(case.v_pool[0])
    tables, ctx, cud = dev(case.block_tables), dev(case.context_lens), dev(cu)
    ops.kv_append(k, v, dev(k_new), dev(v_new), tables, dev(start), cud)
    o, _ = ops.paged_prefill(dev(q), k, v, tables, cud, ctx, int(np.diff(cu).max()), scale=1.0)
    torch.cuda.synchronize()
    assert k.cpu().numpy().tobytes() == kp.tobytes(), f"{what}: K pool after the append"
    assert v.cpu().numpy().tobytes() == vp.tobytes(), f"{what}: V pool after the append"
    _same(o, want, what)
    say(f"  {what}: {int(cu[-1])} query tokens bit-exact")
    assert_no_device_error()


def _chunks(case, chunks, seed):
    rng = np.random.default_rng(seed)
    T = int(sum(chunks))
    hkv, d = case.num_kv_heads, case.head_dim
    x = rng.standard_normal((T, hkv, d)).astype(np.float32)
    y = rng.standard_normal((T, hkv, d)).astype(np.float32)
    if case.kv_dtype == "bf16":
        from workloads import bf16_bits
        x, y = bf16_bits(x), bf16_bits(y)
    cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    start = (case.context_lens - np.asarray(chunks)).astype(np.int32)
    return x, y, cu, start


@pytest.mark.parametrize("kv_dtype,hq,hkv,d", [("bf16", 32, 8, 128), ("bf16", 14, 2, 64),
                                               ("f32", 12, 12, 64), ("f32", 16, 4, 128)])
def test_probe_prefill(kv_dtype, hq, hkv, d):
    """Contexts across the prefill's 256-block id windows, chunks of 1 to 200 tokens
    (including a whole short prompt)."""
    lens = [5200, 4200, 4111, 9000, 300, 64]
    chunks = [100, 37, 200, 1, 64, 64]
    say(f"probe prefill {kv_dtype} {hq}/{hkv}x{d}")
    case = build_case("pfprobe", lens, hq, hkv, d, kv_dtype, seed=hq + d)
    x, y, cu, start = _chunks(case, chunks, seed=d)
    _prefill_probe_run(case, x, y, cu, start, f"prefill {kv_dtype} {hq}/{hkv}x{d}", seed=hq)


def test_probe_chunked_prefill_as_benched():
    """The benched prefill: 16 sequences, a 512-token chunk each over U{0..3584} prior
    tokens, kv_append then paged_prefill; every query row of every sequence."""
    say("probe chunked_prefill as benched")
    pc = chunked_prefill_case(0)
    _prefill_probe_run(pc.case, pc.k_new, pc.v_new, pc.cu_q, pc.start_pos,
                       "chunked_prefill", seed=3)
