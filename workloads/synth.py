"""Seeded synthetic workloads shaped like the pages' decode workloads.

Everything here is input generation: random draws, block-id bookkeeping for
the initial layout, bf16 rounding of the drawn values and NaN poisoning of
slots that no sequence owns. No attention arithmetic lives here.

Random streams (one ``SeedSequence(seed).spawn(5)`` per case, in this order):
lengths, block order, q, K, V. Large arrays are filled in fixed 4 Mi-element
chunks, each from its own child seed, so the values do not depend on how many
threads fill them.

Shapes follow the two model families the pages name (spindle's GPT-2 124M,
Slipstream's Qwen2.5-0.5B) with block size 16 (spindle, "Paging").
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16
F32_QNAN_BITS = np.uint32(0x7FC00000)
BF16_QNAN_BITS = np.uint16(0x7FC0)
_CHUNK = 1 << 22


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _streams(seed: int) -> dict:
    kids = np.random.SeedSequence(seed).spawn(5)
    return dict(zip(("lengths", "blocks", "q", "k", "v"), kids))


def parallel_normal(ss: np.random.SeedSequence, shape) -> np.ndarray:
    """N(0,1) float32 array of ``shape``; chunk i comes from ``ss.spawn(...)[i]``."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, np.float32)
    kids = ss.spawn(max(1, (n + _CHUNK - 1) // _CHUNK))

    def fill(i):
        sl = out[i * _CHUNK:(i + 1) * _CHUNK]
        np.random.default_rng(kids[i]).standard_normal(out=sl, dtype=np.float32)

    if len(kids) == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(len(kids))))
    return out.reshape(shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bits as uint16.

    NaNs map to the canonical quiet NaN 0x7FC0 (sign kept).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.reshape(-1).view(np.uint32)
    out = np.empty(u.size, np.uint16)

    def conv(i):
        sl = slice(i * _CHUNK, (i + 1) * _CHUNK)
        a = u[sl]
        r = (a >> np.uint32(16)) & np.uint32(1)
        r += np.uint32(0x7FFF)
        r += a
        r >>= np.uint32(16)
        nan = (a & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
        if nan.any():
            r[nan] = ((a[nan] >> np.uint32(16)) & np.uint32(0x8000)) | np.uint32(0x7FC0)
        out[sl] = r

    nchunks = max(1, (u.size + _CHUNK - 1) // _CHUNK)
    if nchunks == 1:
        conv(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(conv, range(nchunks)))
    return out.reshape(x.shape)


@dataclass
class DecodeCase:
    """One paged-decode input set (one or more layers sharing block tables).

    q:        [layers, B, Hq, D]            float32, or uint16 bf16 bits
    k_pool:   [layers, NB, Hkv, 16, D]      same dtype as q
    v_pool:   [layers, NB, Hkv, 16, D]
    block_tables: int32 [B, W]  (entries past a sequence's blocks point at a
                                 fully NaN-poisoned spare block)
    context_lens: int32 [B]
    """

    name: str
    kv_dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    context_lens: np.ndarray
    block_tables: np.ndarray
    num_blocks: int
    q: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    scale: np.float32
    block_size: int = BLOCK_SIZE
    poison_block: int = -1
    fork_parent: np.ndarray | None = None  # for fork cases: parent index per sequence
    shared_blocks: int = 0  # number of physical blocks referenced by >1 sequence
    extra: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def layers(self) -> int:
        return int(self.q.shape[0])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def table_width(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def elem_bytes(self) -> int:
        return 4 if self.kv_dtype == "f32" else 2

    def physical_blocks_used(self) -> int:
        ids = set()
        for s in range(self.batch):
            nb = -(-int(self.context_lens[s]) // self.block_size)
            ids.update(int(x) for x in self.block_tables[s, :nb])
        return len(ids)


def _np_dtype(kv_dtype: str):
    if kv_dtype == "f32":
        return np.float32
    if kv_dtype == "bf16":
        return np.uint16
    raise ValueError(kv_dtype)


def _cast(x: np.ndarray, kv_dtype: str) -> np.ndarray:
    return x if kv_dtype == "f32" else bf16_bits(x)


def _poison(pool: np.ndarray, kv_dtype: str, block_ids, slot_from=0):
    """Overwrite pool[:, block_ids, :, slot_from:, :] with quiet NaN bits."""
    if len(block_ids) == 0:
        return
    if kv_dtype == "f32":
        pool.view(np.uint32)[:, block_ids, :, slot_from:, :] = F32_QNAN_BITS
    else:
        pool[:, block_ids, :, slot_from:, :] = BF16_QNAN_BITS


def _layout(rows, block_order, table_width, block_size):
    """Deal ``block_order`` ids to logical blocks; ``rows`` lists, per sequence,
    either an int (number of private blocks) or (shared_ids, n_private)."""
    B = len(rows)
    pos = 0
    ids_per_seq = []
    for r in rows:
        if isinstance(r, tuple):
            shared, npriv = r
            own = [int(x) for x in block_order[pos:pos + npriv]]
            pos += npriv
            ids_per_seq.append(list(shared) + own)
        else:
            own = [int(x) for x in block_order[pos:pos + r]]
            pos += r
            ids_per_seq.append(own)
    if pos >= len(block_order):
        raise ValueError("pool too small: no spare block left to poison")
    poison = int(block_order[pos])
    used = max(1, max(len(x) for x in ids_per_seq))
    W = table_width if table_width is not None else used
    if W < used:
        raise ValueError("table_width smaller than the longest sequence")
    tables = np.full((B, W), poison, np.int32)
    for s, ids in enumerate(ids_per_seq):
        tables[s, :len(ids)] = ids
    unused = np.array([int(x) for x in block_order[pos:]], np.int64)
    return tables, poison, unused


def build_case(name, context_lens, num_q_heads, num_kv_heads, head_dim, kv_dtype, seed,
               layers=1, num_blocks=None, pool_factor=1.2, table_width=None,
               q_scale=1.0, block_size=BLOCK_SIZE, streams=None) -> DecodeCase:
    """Independent sequences, blocks scattered over the pool in seeded random order."""
    ctx = np.asarray(context_lens, np.int32)
    if ctx.ndim != 1 or (ctx < 0).any():
        raise ValueError("context_lens must be a 1-D array of non-negative ints")
    st = streams or _streams(seed)
    nb = [-(-int(n) // block_size) for n in ctx]
    need = sum(nb)
    if num_blocks is None:
        num_blocks = int(math.ceil(pool_factor * need)) + 1
    order = np.random.default_rng(st["blocks"]).permutation(num_blocks)
    tables, poison, unused = _layout(nb, order, table_width, block_size)
    return _fill(name, ctx, tables, num_blocks, poison, unused, num_q_heads, num_kv_heads,
                 head_dim, kv_dtype, layers, st, q_scale, block_size)


def _fill(name, ctx, tables, num_blocks, poison, unused, hq, hkv, d, kv_dtype, layers, st,
          q_scale, block_size, **extra_fields):
    B = ctx.shape[0]
    q = parallel_normal(st["q"], (layers, B, hq, d))
    if q_scale != 1.0:
        q *= np.float32(q_scale)
    k = parallel_normal(st["k"], (layers, num_blocks, hkv, block_size, d))
    v = parallel_normal(st["v"], (layers, num_blocks, hkv, block_size, d))
    q, k, v = _cast(q, kv_dtype), _cast(k, kv_dtype), _cast(v, kv_dtype)
    _poison(k, kv_dtype, unused)
    _poison(v, kv_dtype, unused)
    for s in range(B):
        n = int(ctx[s])
        r = n % block_size
        if r:
            last = int(tables[s, n // block_size])
            _poison(k, kv_dtype, [last], r)
            _poison(v, kv_dtype, [last], r)
    return DecodeCase(name=name, kv_dtype=kv_dtype, num_q_heads=hq, num_kv_heads=hkv,
                      head_dim=d, context_lens=ctx, block_tables=tables,
                      num_blocks=int(num_blocks), q=q, k_pool=k, v_pool=v,
                      scale=np.float32(1.0 / math.sqrt(d)), block_size=block_size,
                      poison_block=poison, **extra_fields)


def fork_case(name, prefix_lens, forks_per_parent, private_lens, num_q_heads, num_kv_heads,
              head_dim, kv_dtype, seed, pool_factor=1.2, num_blocks=None,
              block_size=BLOCK_SIZE, streams=None) -> DecodeCase:
    """Parents' prefixes held once and shared by their forks (copy-on-write layout).

    Fork f of parent p attends to p's prefix blocks followed by its own private
    blocks.  A prefix that is not block-aligned is only allowed with no private
    tokens (a private token would have to land in a copied block).
    """
    st = streams or _streams(seed)
    prefix_lens = [int(x) for x in prefix_lens]
    P = len(prefix_lens)
    if np.ndim(forks_per_parent) == 0:
        forks = [int(forks_per_parent)] * P
        private_lens = np.asarray(private_lens, np.int64).reshape(P, forks[0]).tolist()
    else:  # one fork count per parent, private_lens ragged to match
        forks = [int(f) for f in forks_per_parent]
        private_lens = [[int(x) for x in row] for row in private_lens]
        if [len(r) for r in private_lens] != forks:
            raise ValueError("private_lens rows must match forks_per_parent")
    for p in range(P):
        if prefix_lens[p] % block_size and any(x > 0 for x in private_lens[p]):
            raise ValueError("unaligned prefix with private tokens needs a CoW copy")
    pref_nb = [-(-n // block_size) for n in prefix_lens]
    priv_nb = [[-(-int(x) // block_size) for x in row] for row in private_lens]
    need = sum(pref_nb) + sum(sum(r) for r in priv_nb)
    if num_blocks is None:
        num_blocks = int(math.ceil(pool_factor * need)) + 1
    order = np.random.default_rng(st["blocks"]).permutation(num_blocks)
    pos = 0
    prefix_ids = []
    for nb in pref_nb:
        prefix_ids.append([int(x) for x in order[pos:pos + nb]])
        pos += nb
    rows, ctx, parent = [], [], []
    for p in range(P):
        for f in range(forks[p]):
            rows.append((prefix_ids[p], priv_nb[p][f]))
            ctx.append(prefix_lens[p] + int(private_lens[p][f]))
            parent.append(p)
    tables, poison, unused = _layout(rows, order[pos:], None, block_size)
    ctx = np.asarray(ctx, np.int32)
    case = _fill(name, ctx, tables, num_blocks, poison, unused, num_q_heads, num_kv_heads,
                 head_dim, kv_dtype, 1, st, 1.0, block_size,
                 fork_parent=np.asarray(parent, np.int32),
                 shared_blocks=sum(nb for nb, f in zip(pref_nb, forks) if f > 1))
    return case


def fork_groups(case: DecodeCase):
    """Group layout of a fork case: (group_starts int32 [G + 1], shared_blocks int32 [G]).

    Members of a group are consecutive sequences with the same parent; a group's shared
    count is the length of the run of leading block ids that all its members' tables hold
    in common (over the blocks each member uses)."""
    if case.fork_parent is None:
        raise ValueError("not a fork case")
    parent = case.fork_parent.tolist()
    starts = [0] + [s for s in range(1, len(parent)) if parent[s] != parent[s - 1]]
    starts.append(len(parent))
    shared = []
    for g in range(len(starts) - 1):
        rows = range(starts[g], starts[g + 1])
        used = min(-(-int(case.context_lens[s]) // BLOCK_SIZE) for s in rows)
        k = 0
        while k < used and len({int(case.block_tables[s, k]) for s in rows}) == 1:
            k += 1
        shared.append(k)
    return np.asarray(starts, np.int32), np.asarray(shared, np.int32)


def block_refcounts(case: DecodeCase) -> dict:
    """Physical block id -> number of sequences whose used blocks include it."""
    refs = {}
    for s, n in enumerate(case.context_lens.tolist()):
        for j in range(-(-n // BLOCK_SIZE)):
            b = int(case.block_tables[s, j])
            refs[b] = refs.get(b, 0) + 1
    return refs


# --------------------------------------------------------------------------------------
# The five workload shapes.  Distribution parameters the pages leave open are fixed
# here (lognormal sigma = ln 2 so that the stated maximum is 8x the median, i.e. e^(3 sigma)).
# --------------------------------------------------------------------------------------

CONFIGS = {
    # GPT-2 124M head shape, fp32, 4 sequences, 64-block pool
    "tiny": dict(kv_dtype="f32", hq=12, hkv=12, d=64, batch=4, layers=1),
    # GPT-2 124M replay, fp32, 12 layers, 24 sequences, 8192-token pool
    "gpt2_replay": dict(kv_dtype="f32", hq=12, hkv=12, d=64, batch=24, layers=12),
    # Qwen2.5-0.5B attention shape, bf16 K/V, 14 q heads over 2 KV heads, 24 layers
    "qwen_gqa": dict(kv_dtype="bf16", hq=14, hkv=2, d=64, batch=64, layers=24),
    # bandwidth-bound decode, bf16, 32 q heads over 8 KV heads, head_dim 128, 256 seqs
    "high_concurrency": dict(kv_dtype="bf16", hq=32, hkv=8, d=128, batch=256, layers=1),
    # 16 parents x 2048-token prefix, forked 4 ways, plus 0..256 private tokens
    "prefix_fork": dict(kv_dtype="bf16", hq=32, hkv=8, d=128, batch=64, layers=1),
    # 4 sequences of 32768 tokens, split-KV partitions of 512
    "long_context": dict(kv_dtype="bf16", hq=32, hkv=8, d=128, batch=4, layers=1,
                         partition_size=512),
}


def _lognormal_lengths(rng, n, median, sigma, hi):
    x = np.exp(rng.normal(math.log(median), sigma, n))
    return np.clip(np.rint(x), 1, hi).astype(np.int32)


def config_lengths(name: str, seed: int) -> np.ndarray:
    rng = np.random.default_rng(_streams(seed)["lengths"])
    if name == "tiny":
        return rng.integers(1, 193, size=4).astype(np.int32)
    if name == "qwen_gqa":
        return _lognormal_lengths(rng, 64, 512, math.log(2.0), 4096)
    if name == "high_concurrency":
        return _lognormal_lengths(rng, 256, 1024, math.log(2.0), 8192)
    if name == "long_context":
        return np.full(4, 32768, np.int32)
    raise ValueError(f"no length recipe for {name!r}")


def config_case(name: str, seed: int = 0, layers: int | None = None, q_scale: float = 1.0,
                max_batch: int | None = None) -> DecodeCase:
    """Build the named workload.  ``layers`` may cut a multi-layer shape down
    (tests); ``max_batch`` keeps only the first sequences (bounded samples)."""
    cfg = CONFIGS[name]
    st = _streams(seed)
    nl = cfg["layers"] if layers is None else layers
    if name == "prefix_fork":
        rng = np.random.default_rng(st["lengths"])
        priv = rng.integers(0, 257, size=64)
        case = fork_case(name, [2048] * 16, 4, priv, cfg["hq"], cfg["hkv"], cfg["d"],
                         cfg["kv_dtype"], seed, streams=st)
        return case
    if name == "gpt2_replay":
        raise ValueError("gpt2_replay is a multi-step replay: use replay_schedule()")
    ctx = config_lengths(name, seed)
    if max_batch is not None:
        ctx = ctx[:max_batch]
    num_blocks = 64 if name == "tiny" else None
    case = build_case(name, ctx, cfg["hq"], cfg["hkv"], cfg["d"], cfg["kv_dtype"], seed,
                      layers=nl, num_blocks=num_blocks, q_scale=q_scale, streams=st)
    if "partition_size" in cfg:
        case.extra["partition_size"] = cfg["partition_size"]
    return case


# --------------------------------------------------------------------------------------
# GPT-2-shaped continuous-batching replay: 24 sequences admitted together, prompt
# appended as one multi-token write per layer, then one token per step per layer.
# A sequence leaves (its blocks return to the pool) after its last generated token.
# --------------------------------------------------------------------------------------

@dataclass
class ReplaySchedule:
    seed: int
    prompt_lens: np.ndarray
    gen_lens: np.ndarray
    free_order: np.ndarray          # initial free-list order of the pool's block ids
    num_blocks: int = 512           # 8192 token slots
    layers: int = 12
    num_q_heads: int = 12
    num_kv_heads: int = 12
    head_dim: int = 64
    block_size: int = BLOCK_SIZE

    @property
    def batch(self) -> int:
        return int(self.prompt_lens.shape[0])

    @property
    def steps(self) -> int:
        return int(self.gen_lens.max())


def replay_schedule(seed: int = 0, batch: int = 24, layers: int = 12) -> ReplaySchedule:
    st = _streams(seed)
    rng = np.random.default_rng(st["lengths"])
    prompts = rng.integers(16, 129, size=batch).astype(np.int32)
    gens = _lognormal_lengths(rng, batch, 48, 0.75, 192)
    order = np.random.default_rng(st["blocks"]).permutation(512).astype(np.int32)
    return ReplaySchedule(seed=seed, prompt_lens=prompts, gen_lens=gens, free_order=order,
                          layers=layers)


def replay_step_values(sched: ReplaySchedule, step: int, layer: int, seqs, kind: str):
    """Values for one replay step (step -1 = the prompt) and layer.

    kind 'kv' -> (k_new, v_new) float32 [T, Hkv, D] for the listed sequences
    (T = sum of prompt lengths at step -1, else one token each);
    kind 'q'  -> q float32 [len(seqs), Hq, D].
    """
    tag = {"kv": 1, "q": 2}[kind]
    ss = np.random.SeedSequence(entropy=sched.seed, spawn_key=(7, tag, step + 1, layer))
    if kind == "q":
        return parallel_normal(ss, (len(seqs), sched.num_q_heads, sched.head_dim))
    T = int(sum(int(sched.prompt_lens[s]) for s in seqs)) if step < 0 else len(seqs)
    ks, vs = ss.spawn(2)
    k = parallel_normal(ks, (T, sched.num_kv_heads, sched.head_dim))
    v = parallel_normal(vs, (T, sched.num_kv_heads, sched.head_dim))
    return k, v


# --------------------------------------------------------------------------------------
# Allocator replay: 64 requests through an 8192-slot cache with 16-token blocks, prompt
# and generation lengths drawn as in the GPT-2 replay; max_new_tokens 192 (the bound a
# contiguous buffer must be sized for at admission).
# --------------------------------------------------------------------------------------

def allocator_replay_requests(seed: int = 0, n: int = 64):
    """(prompt_lens, gen_lens) int32 [n] and the settings of the replay."""
    st = _streams(seed)
    rng = np.random.default_rng(st["lengths"])
    prompts = rng.integers(16, 129, size=n).astype(np.int32)
    gens = _lognormal_lengths(rng, n, 48, 0.75, 192)
    return prompts, gens, dict(max_new_tokens=192, total_slots=8192, block_size=16)


# --------------------------------------------------------------------------------------
# Chunked prefill: 16 sequences each append a 512-token chunk onto a prior context of
# U{0..3584} tokens and attend it causally (bf16, 32/8 heads, head_dim 128).
# --------------------------------------------------------------------------------------

@dataclass
class PrefillCase:
    case: DecodeCase          # pools and tables for the full contexts (prior + chunk)
    q: np.ndarray             # [T, Hq, D] query rows of the chunks, bf16 bits
    k_new: np.ndarray         # [T, Hkv, D] the chunks' K, bf16 bits
    v_new: np.ndarray
    cu_q: np.ndarray          # int32 [B + 1]
    start_pos: np.ndarray     # int32 [B]: each chunk's first position (the prior length)


def chunked_prefill_case(seed: int = 0, batch: int = 16, chunk: int = 512,
                         max_prior: int = 3584, hq: int = 32, hkv: int = 8,
                         d: int = 128) -> PrefillCase:
    st = _streams(seed)
    rng = np.random.default_rng(st["lengths"])
    prior = rng.integers(0, max_prior + 1, size=batch).astype(np.int32)
    ctx = (prior + chunk).astype(np.int32)
    case = build_case("chunked_prefill", ctx, hq, hkv, d, "bf16", seed, streams=st)
    kids = np.random.SeedSequence(entropy=seed, spawn_key=(77,)).spawn(3)
    T = batch * chunk
    q = bf16_bits(parallel_normal(kids[0], (T, hq, d)))
    k_new = bf16_bits(parallel_normal(kids[1], (T, hkv, d)))
    v_new = bf16_bits(parallel_normal(kids[2], (T, hkv, d)))
    cu = (np.arange(batch + 1) * chunk).astype(np.int32)
    return PrefillCase(case, q, k_new, v_new, cu, prior)


# --------------------------------------------------------------------------------------
# The decode step's new tokens: one per sequence at position ctx - 1 (the context counts
# the token appended this step).  Copy-on-write: a token is never written into a block
# that several sequences hold (a fork with no private token would first copy it), so such
# sequences append nothing this step.
# --------------------------------------------------------------------------------------

@dataclass
class StepInputs:
    k_new: np.ndarray      # [T, Hkv, D] cache dtype
    v_new: np.ndarray
    start_pos: np.ndarray  # int32 [B]
    cu_new: np.ndarray     # int32 [B + 1]


def decode_step_inputs(case: DecodeCase, seed: int) -> StepInputs:
    B, hkv, d = case.batch, case.num_kv_heads, case.head_dim
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(99,))
    kn = parallel_normal(ss.spawn(1)[0], (B, hkv, d))
    vn = parallel_normal(ss.spawn(1)[0], (B, hkv, d))
    if case.kv_dtype == "bf16":
        kn, vn = bf16_bits(kn), bf16_bits(vn)
    start = (case.context_lens - 1).clip(min=0).astype(np.int32)
    counts = (case.context_lens > 0).astype(np.int32)
    if case.shared_blocks:
        refs = block_refcounts(case)
        for s in range(B):
            if counts[s] and refs[int(case.block_tables[s, start[s] // BLOCK_SIZE])] > 1:
                counts[s] = 0
    cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return StepInputs(kn[counts > 0], vn[counts > 0], start, cu)
