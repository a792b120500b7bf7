"""Checks that pin the CPU oracle to things other than itself.

Each ``check_*`` takes the oracle module under test (``oracle.paged_attention``
or ``oracle.block_pool``, or a deliberately broken copy of one) and raises
AssertionError when it disagrees with a closed form, a library routine, brute
force, an invariant of the method or a fixture holding the pages' worked
example.  ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutants.py`` plants mistakes in copies of the oracle's source
and requires every mutant to be caught by at least one check.
"""

from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np

from oracle import brute
from workloads import bf16_bits, build_case, fork_case

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
BS = 16


def _close(a, b, tol=1e-12, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin), f"{what}: finiteness differs"
    assert np.array_equal(a[~fin], b[~fin]), f"{what}: infinities differ"
    if fin.any():
        err = np.max(np.abs(a[fin] - b[fin]) / np.maximum(1.0, np.abs(b[fin])))
        assert err <= tol, f"{what}: rel err {err:.3e} > {tol}"


def _widen(x, kv_dtype):
    """Test-side exact decoding of stored values (independent of the oracle's)."""
    if kv_dtype == "f32":
        return np.asarray(x, np.float32).astype(np.float64)
    out = np.zeros(np.shape(x), np.float64)
    flat = np.asarray(x, np.uint16).reshape(-1)
    of = out.reshape(-1)
    for i, b in enumerate(flat.tolist()):  # sign, exponent, mantissa by hand
        sign = -1.0 if b & 0x8000 else 1.0
        e = (b >> 7) & 0xFF
        m = b & 0x7F
        if e == 0xFF:
            of[i] = math.nan if m else sign * math.inf
        elif e == 0:
            of[i] = sign * m * 2.0 ** (-133)
        else:
            of[i] = sign * (1.0 + m / 128.0) * 2.0 ** (e - 127)
    return out


def _rand(rng, shape, kv_dtype):
    x = rng.standard_normal(shape).astype(np.float32)
    return x if kv_dtype == "f32" else bf16_bits(x)


def _scatter(contig_k, contig_v, num_blocks, rng, kv_dtype, hkv, d):
    """Place per-sequence contiguous [Hkv, n, D] arrays into a NaN pool via a random table."""
    dt = np.float32 if kv_dtype == "f32" else np.uint16
    kp = np.empty((num_blocks, hkv, BS, d), dt)
    vp = np.empty_like(kp)
    if kv_dtype == "f32":
        kp.view(np.uint32)[:] = 0x7FC00000
        vp.view(np.uint32)[:] = 0x7FC00000
    else:
        kp[:] = 0x7FC0
        vp[:] = 0x7FC0
    order = rng.permutation(num_blocks)
    nbs = [-(-k.shape[1] // BS) for k in contig_k]
    W = max(1, max(nbs))
    tables = np.full((len(contig_k), W), order[-1], np.int32)
    pos = 0
    for s, (K, V) in enumerate(zip(contig_k, contig_v)):
        for t in range(K.shape[1]):
            if t % BS == 0:
                tables[s, t // BS] = order[pos]
                pos += 1
            b = tables[s, t // BS]
            kp[b, :, t % BS, :] = K[:, t, :]
            vp[b, :, t % BS, :] = V[:, t, :]
    assert pos < num_blocks
    return kp, vp, tables


# ---------------------------------------------------------------------------------------
# P-a: paged == contiguous
# ---------------------------------------------------------------------------------------

def check_gather_roundtrip(pa, kv_dtype="f32", seed=0, hkv=3, d=8):
    rng = np.random.default_rng(seed)
    lens = [0, 1, 15, 16, 17, 33, 47, 80]
    Ks = [_rand(rng, (hkv, n, d), kv_dtype) for n in lens]
    Vs = [_rand(rng, (hkv, n, d), kv_dtype) for n in lens]
    kp, vp, tables = _scatter(Ks, Vs, 40, rng, kv_dtype, hkv, d)
    for s, n in enumerate(lens):
        gk = pa.gather_sequence(kp, tables[s], n, BS)
        gv = pa.gather_sequence(vp, tables[s], n, BS)
        assert gk.shape == Ks[s].shape
        assert gk.tobytes() == Ks[s].tobytes(), f"gather K not bitwise (n={n})"
        assert gv.tobytes() == Vs[s].tobytes(), f"gather V not bitwise (n={n})"


def check_paged_vs_contiguous(pa, kv_dtype="f32", seed=1, hq=6, hkv=2, d=16):
    rng = np.random.default_rng(seed)
    lens = [1, 5, 16, 17, 40, 64, 100]
    Ks = [_rand(rng, (hkv, n, d), kv_dtype) for n in lens]
    Vs = [_rand(rng, (hkv, n, d), kv_dtype) for n in lens]
    q = _rand(rng, (len(lens), hq, d), kv_dtype)
    kp, vp, tables = _scatter(Ks, Vs, 64, rng, kv_dtype, hkv, d)
    scale = np.float32(1 / math.sqrt(d))
    o1, l1 = pa.paged_decode(q, kp, vp, tables, np.array(lens, np.int32), scale, kv_dtype)
    o2, l2 = pa.contiguous_decode(q, Ks, Vs, scale, kv_dtype)
    _close(o1, o2, 1e-12, "paged vs contiguous out")
    _close(l1, l2, 1e-12, "paged vs contiguous lse")


# ---------------------------------------------------------------------------------------
# P-b: closed forms
# ---------------------------------------------------------------------------------------

def _single(pa, q, K, V, scale, kv_dtype="f32"):
    """Run the paged oracle on one sequence given contiguous K/V [Hkv, n, D]."""
    rng = np.random.default_rng(123)
    hkv, n, d = K.shape
    kp, vp, tables = _scatter([K], [V], -(-n // BS) + 3, rng, kv_dtype, hkv, d)
    return pa.paged_decode(q[None], kp, vp, tables, np.array([n], np.int32), scale, kv_dtype)


def check_closed_forms(pa):
    rng = np.random.default_rng(7)
    d = 8
    # one token: softmax weight is exactly 1, out = v0, lse = score
    q = rng.standard_normal((1, d)).astype(np.float32)
    K = rng.standard_normal((1, 1, d)).astype(np.float32)
    V = rng.standard_normal((1, 1, d)).astype(np.float32)
    scale = np.float32(0.3535533905932738)
    o, l = _single(pa, q, K, V, scale)
    assert np.array_equal(o[0, 0], V[0, 0].astype(np.float64)), "ctx=1: out != v0"
    s0 = float(scale) * math.fsum(float(a) * float(b) for a, b in zip(q[0], K[0, 0]))
    _close(l[0, 0], s0, 1e-14, "ctx=1 lse")

    # two tokens with a score gap of x: weights 1/(1+e^x), e^x/(1+e^x)
    x = np.float32(math.log(3.0))
    q = np.zeros((1, 2), np.float32); q[0, 0] = 1
    K = np.array([[[0.0, 5.0], [x, -7.0]]], np.float32)
    V = np.array([[[4.0, 8.0], [0.0, -4.0]]], np.float32)
    o, l = _single(pa, q, K, V, np.float32(1.0))
    ex = math.exp(float(x))
    want = [(4.0 + ex * 0.0) / (1 + ex), (8.0 - 4.0 * ex) / (1 + ex)]
    _close(o[0, 0], want, 1e-14, "two-token out")
    _close(l[0, 0], math.log(1 + ex), 1e-14, "two-token lse")

    # identical keys: uniform weights, out = mean(V), lse = s + ln n, for any q
    n = 37
    k = rng.standard_normal(d).astype(np.float32)
    K = np.broadcast_to(k, (1, n, d)).copy()
    V = rng.standard_normal((1, n, d)).astype(np.float32)
    q = rng.standard_normal((1, d)).astype(np.float32)
    o, l = _single(pa, q, K, V, np.float32(0.25))
    _close(o[0, 0], V[0].astype(np.float64).mean(axis=0), 1e-13, "equal keys out")
    s = 0.25 * math.fsum(float(a) * float(b) for a, b in zip(q[0], k))
    _close(l[0, 0], s + math.log(n), 1e-13, "equal keys lse")

    # q = 0: uniform weights, lse = ln n
    q = np.zeros((1, d), np.float32)
    K = rng.standard_normal((1, n, d)).astype(np.float32)
    o, l = _single(pa, q, K, V, np.float32(0.25))
    _close(o[0, 0], V[0].astype(np.float64).mean(axis=0), 1e-13, "q=0 out")
    _close(l[0, 0], math.log(n), 1e-13, "q=0 lse")

    # one-hot: token j's score exceeds every other by >= 100 -> out = V[j]
    n = 50
    j = 29
    K = rng.standard_normal((1, n, d)).astype(np.float32) * np.float32(0.1)
    K[0, j] = 0
    K[0, j, 0] = 40.0
    q = np.zeros((1, d), np.float32); q[0, 0] = 4.0
    V = rng.standard_normal((1, n, d)).astype(np.float32)
    o, l = _single(pa, q, K, V, np.float32(1.0))
    _close(o[0, 0], V[0, j].astype(np.float64), 1e-30, "one-hot out")
    _close(l[0, 0], 160.0, 1e-15, "one-hot lse")

    # empty context: out = 0, lse = -inf
    kp = np.zeros((2, 1, BS, d), np.float32)
    o, l = pa.paged_decode(np.ones((1, 1, d), np.float32), kp, kp, np.zeros((1, 1), np.int32),
                           np.array([0], np.int32), np.float32(1.0), "f32")
    assert np.all(o == 0) and l[0, 0] == -np.inf


# ---------------------------------------------------------------------------------------
# P-c: a library routine on the contiguous special case
# ---------------------------------------------------------------------------------------

def check_library_sdpa(pa, kv_dtype="bf16", seed=3):
    import torch
    import torch.nn.functional as F
    case = build_case("sdpa", [1, 9, 16, 31, 77, 130], 8, 2, 32, kv_dtype, seed)
    o, l = pa.paged_decode(case.q[0], case.k_pool[0], case.v_pool[0], case.block_tables,
                           case.context_lens, case.scale, kv_dtype)
    G = case.group
    for s, n in enumerate(case.context_lens.tolist()):
        ids = case.block_tables[s, :-(-n // BS)]
        K = _widen(case.k_pool[0][ids], kv_dtype).transpose(1, 0, 2, 3).reshape(2, -1, 32)[:, :n]
        V = _widen(case.v_pool[0][ids], kv_dtype).transpose(1, 0, 2, 3).reshape(2, -1, 32)[:, :n]
        Kt = torch.from_numpy(np.ascontiguousarray(K)).repeat_interleave(G, dim=0)
        Vt = torch.from_numpy(np.ascontiguousarray(V)).repeat_interleave(G, dim=0)
        qt = torch.from_numpy(_widen(case.q[0, s], kv_dtype))[:, None, :]
        ref = F.scaled_dot_product_attention(qt, Kt, Vt, scale=float(case.scale))[:, 0]
        scores = (qt @ Kt.transpose(1, 2))[:, 0] * float(case.scale)
        ref_lse = torch.logsumexp(scores, dim=-1)
        _close(o[s], ref.numpy(), 1e-12, "sdpa out")
        _close(l[s], ref_lse.numpy(), 1e-12, "sdpa lse")


# ---------------------------------------------------------------------------------------
# P-d: invariants of the method
# ---------------------------------------------------------------------------------------

def check_permutation_invariance(pa, kv_dtype="f32", seed=4):
    case = build_case("perm", [3, 16, 29, 50, 64], 4, 2, 16, kv_dtype, seed)
    args = (case.context_lens, case.scale, kv_dtype)
    o1, l1 = pa.paged_decode(case.q[0], case.k_pool[0], case.v_pool[0], case.block_tables, *args)
    perm = np.random.default_rng(seed).permutation(case.num_blocks)
    kp = np.empty_like(case.k_pool[0]); kp[perm] = case.k_pool[0]
    vp = np.empty_like(case.v_pool[0]); vp[perm] = case.v_pool[0]
    o2, l2 = pa.paged_decode(case.q[0], kp, vp, perm[case.block_tables].astype(np.int32), *args)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2), "pool permutation changed output"


def check_batched_equals_alone(pa, kv_dtype="bf16", seed=5):
    case = build_case("alone", [7, 33, 1, 90, 48], 6, 3, 16, kv_dtype, seed)
    o, l = pa.paged_decode(case.q[0], case.k_pool[0], case.v_pool[0], case.block_tables,
                           case.context_lens, case.scale, kv_dtype)
    for s in range(case.batch):
        o1, l1 = pa.paged_decode(case.q[0, s:s + 1], case.k_pool[0], case.v_pool[0],
                                 case.block_tables[s:s + 1], case.context_lens[s:s + 1],
                                 case.scale, kv_dtype)
        assert np.array_equal(o1[0], o[s]) and np.array_equal(l1[0], l[s]), f"seq {s} leaks"


def check_forks_identical(pa, kv_dtype="bf16", seed=6):
    case = fork_case("forks", [20, 32], 4, [[0] * 4, [0, 0, 0, 0]], 4, 2, 16, kv_dtype, seed)
    q = case.q[0].copy()
    for s in range(case.batch):
        q[s] = q[case.fork_parent[s] * 4]
    o, l = pa.paged_decode(q, case.k_pool[0], case.v_pool[0], case.block_tables,
                           case.context_lens, case.scale, kv_dtype)
    for s in range(case.batch):
        f0 = case.fork_parent[s] * 4
        assert np.array_equal(o[s], o[f0]) and np.array_equal(l[s], l[f0]), "forks differ"
    # a fork with private tokens must differ from its parent's output
    case2 = fork_case("forks2", [32], 2, [[0, 5]], 4, 2, 16, kv_dtype, seed)
    q2 = case2.q[0].copy(); q2[1] = q2[0]
    o2, _ = pa.paged_decode(q2, case2.k_pool[0], case2.v_pool[0], case2.block_tables,
                            case2.context_lens, case2.scale, kv_dtype)
    assert not np.array_equal(o2[0], o2[1]), "private tokens ignored"


def check_append(pa, kv_dtype="f32", seed=8, hkv=2, d=8):
    rng = np.random.default_rng(seed)
    nb = 12
    dt = np.float32 if kv_dtype == "f32" else np.uint16
    kp = _rand(rng, (nb, hkv, BS, d), kv_dtype).astype(dt)
    vp = _rand(rng, (nb, hkv, BS, d), kv_dtype).astype(dt)
    tables = rng.permutation(nb)[:9].reshape(3, 3).astype(np.int32)
    starts = np.array([14, 0, 31], np.int32)     # crosses a block edge / first slot / edge
    counts = [5, 1, 9]
    cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    kn = _rand(rng, (cu[-1], hkv, d), kv_dtype).astype(dt)
    vn = _rand(rng, (cu[-1], hkv, d), kv_dtype).astype(dt)
    k2, v2 = pa.kv_append(kp, vp, kn, vn, tables, starts, cu)
    # expected: brute-force per-position writes on nested lists of raw bits
    expect_k = kp.copy(); expect_v = vp.copy()
    target = np.zeros((nb, hkv, BS), bool)
    for s in range(3):
        for i in range(counts[s]):
            p = int(starts[s]) + i
            b, slot = brute.token_location(tables[s].tolist(), p)
            expect_k[b, :, slot] = kn[cu[s] + i]
            expect_v[b, :, slot] = vn[cu[s] + i]
            target[b, :, slot] = True
    assert k2.tobytes() == expect_k.tobytes(), "append K bits wrong"
    assert v2.tobytes() == expect_v.tobytes(), "append V bits wrong"
    changed = (k2.view(np.uint8).reshape(nb, hkv, BS, -1) != kp.view(np.uint8).reshape(
        nb, hkv, BS, -1)).any(-1)
    assert not (changed & ~target).any(), "append touched a slot outside its range"
    assert kp.tobytes() != k2.tobytes()


def check_copy_blocks(pa, seed=9):
    rng = np.random.default_rng(seed)
    kp = rng.standard_normal((6, 2, BS, 4)).astype(np.float32)
    vp = rng.standard_normal((6, 2, BS, 4)).astype(np.float32)
    k2, v2 = pa.copy_blocks(kp, vp, [1, 4], [3, 0])
    for b, src in [(0, 4), (1, 1), (2, 2), (3, 1), (4, 4), (5, 5)]:
        assert k2[b].tobytes() == kp[src].tobytes() and v2[b].tobytes() == vp[src].tobytes()


# ---------------------------------------------------------------------------------------
# P-e: split identity
# ---------------------------------------------------------------------------------------

def check_split_identity(pa, kv_dtype="f32", seed=10, q_scale=1.0):
    case = build_case("split", [0, 1, 15, 16, 17, 95, 200, 333], 4, 2, 16, kv_dtype, seed,
                      q_scale=q_scale)
    args = (case.q[0], case.k_pool[0], case.v_pool[0], case.block_tables, case.context_lens,
            case.scale, kv_dtype)
    o, l = pa.paged_decode(*args)
    for P in (16, 32, 48, 64, 512):
        po, pl = pa.decode_partitions(*args, P)
        assert po.shape[2] == max(1, -(-int(case.context_lens.max()) // P))
        o2, l2 = pa.combine_partitions(po, pl)
        _close(o2, o, 1e-12, f"split P={P} out")
        _close(l2, l, 1e-12, f"split P={P} lse")
        for s, n in enumerate(case.context_lens.tolist()):
            npart = -(-n // P)
            assert np.all(pl[s, :, npart:] == -np.inf) and np.all(po[s, :, npart:] == 0)
    # one partition covering everything is the unsplit result itself
    po, pl = pa.decode_partitions(*args, 512)
    assert np.array_equal(po[:, :, 0], o) and np.array_equal(pl[:, :, 0], l)
    oc, lc = pa.combine_partitions(po[:, :, :1], pl[:, :, :1])
    assert np.array_equal(oc, o) and np.array_equal(lc, l)


# ---------------------------------------------------------------------------------------
# P-f: brute force on tiny inputs
# ---------------------------------------------------------------------------------------

def _as_lists(case, kv_dtype):
    return (_widen(case.q[0], kv_dtype).tolist(), _widen(case.k_pool[0], kv_dtype).tolist(),
            _widen(case.v_pool[0], kv_dtype).tolist())


def check_brute_force(pa, seed=11):
    for d, (hq, hkv), kv_dtype in [(1, (1, 1), "f32"), (2, (2, 1), "bf16"),
                                   (8, (3, 1), "f32"), (8, (4, 2), "bf16")]:
        lens = [0, 1, 2, 15, 16, 17, 31, 32, 33, 48]
        case = build_case("brute", lens, hq, hkv, d, kv_dtype, seed + d)
        o, l = pa.paged_decode(case.q[0], case.k_pool[0], case.v_pool[0], case.block_tables,
                               case.context_lens, case.scale, kv_dtype)
        ql, kl, vl = _as_lists(case, kv_dtype)
        ob, lb = brute.decode(ql, kl, vl, case.block_tables.tolist(), lens, float(case.scale))
        _close(o, ob, 1e-12, f"brute out d={d}")
        _close(l, lb, 1e-12, f"brute lse d={d}")
        po, pl = pa.decode_partitions(case.q[0], case.k_pool[0], case.v_pool[0],
                                      case.block_tables, case.context_lens, case.scale,
                                      kv_dtype, 16)
        oc, lc = pa.combine_partitions(po, pl)
        for s in range(len(lens)):
            for h in range(hq):
                bo, bl = brute.combine(po[s, h].tolist(), pl[s, h].tolist())
                _close(oc[s, h], bo, 1e-12, "brute combine out")
                _close(lc[s, h], bl, 1e-12, "brute combine lse")


def check_all_pool_permutations(pa, seed=12):
    """A 4-block pool under every block placement gives the brute-force answer."""
    rng = np.random.default_rng(seed)
    d, n = 2, 40
    base_k = rng.standard_normal((4, 1, BS, d)).astype(np.float32)
    base_v = rng.standard_normal((4, 1, BS, d)).astype(np.float32)
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    ref = None
    for perm in itertools.permutations(range(4)):
        kp = np.empty_like(base_k); vp = np.empty_like(base_v)
        kp[list(perm)] = base_k; vp[list(perm)] = base_v
        table = np.array([[perm[0], perm[1], perm[2]]], np.int32)
        o, l = pa.paged_decode(q, kp, vp, table, np.array([n], np.int32), np.float32(0.7), "f32")
        ob, lb = brute.decode(q.astype(np.float64).tolist(), kp.astype(np.float64).tolist(),
                              vp.astype(np.float64).tolist(), table.tolist(), [n], float(np.float32(0.7)))
        _close(o, ob, 1e-12, "perm brute out")
        _close(l, lb, 1e-12, "perm brute lse")
        if ref is None:
            ref = (o, l)
        assert np.array_equal(ref[0], o) and np.array_equal(ref[1], l)


# ---------------------------------------------------------------------------------------
# Block pool: the pages' worked example and the copy-on-write rules
# ---------------------------------------------------------------------------------------

def check_cow_golden(bp):
    g = json.load(open(os.path.join(GOLDEN, "cow_fork_example.json")))
    pool = bp.BlockPool(8, g["block_size"])
    parent = pool.add_sequence()
    assert pool.prepare_write(parent, 0, g["parent_tokens"]) == []
    seqs = [parent] + [pool.fork(parent) for _ in range(g["sequences_total"] - 1)]
    logical = g["parent_tokens"] * len(seqs)
    physical = pool.physical_in_use()
    assert logical == g["expected_logical_tokens"]
    assert physical == g["expected_physical_blocks"]
    assert physical * g["block_size"] == g["expected_physical_slots"]
    b = pool.table(parent)[0]
    assert all(pool.table(s) == [b] for s in seqs)
    assert pool.refcount[b] == g["expected_refcount"]
    # retiring all four returns the block
    for s in seqs:
        pool.free_sequence(s)
    assert pool.num_free() == 8 and pool.refcount[b] == 0


def check_cow_write(bp):
    pool = bp.BlockPool(10, 16, free_order=[5, 2, 9, 0, 1, 3, 4, 6, 7, 8])
    p = pool.add_sequence()
    assert pool.prepare_write(p, 0, 20) == []          # blocks 5, 2
    assert pool.table(p) == [5, 2]
    c = pool.fork(p)
    assert pool.refcount[5] == 2 and pool.refcount[2] == 2
    # child writes position 20 (inside shared block 2): copy 2 -> 9 first
    assert pool.prepare_write(c, 20, 1) == [(2, 9)]
    assert pool.table(c) == [5, 9] and pool.table(p) == [5, 2]
    assert pool.refcount[2] == 1 and pool.refcount[9] == 1 and pool.refcount[5] == 2
    # parent writes position 20 now: block 2 is its own, no copy
    assert pool.prepare_write(p, 20, 1) == []
    # growing past the table takes fresh blocks in FIFO order
    assert pool.prepare_write(c, 21, 12) == []        # positions 21..32 -> block idx 2 new
    assert pool.table(c) == [5, 9, 0]
    pool.free_sequence(p)                               # 5 stays (child), 2 freed
    assert pool.refcount[5] == 1 and list(pool.free)[-1] == 2
    # the pool is exhausted atomically
    small = bp.BlockPool(2, 16)
    s = small.add_sequence()
    try:
        small.prepare_write(s, 0, 48)
    except bp.OutOfBlocks:
        pass
    else:
        raise AssertionError("expected OutOfBlocks")
    assert small.num_free() == 2 and small.table(s) == []


def check_waste_bound(bp, seed=13):
    g = json.load(open(os.path.join(GOLDEN, "paging_waste_bound.json")))
    rng = np.random.default_rng(seed)
    pool = bp.BlockPool(512, g["block_size"], free_order=rng.permutation(512))
    lens = {}
    for _ in range(40):
        s = pool.add_sequence()
        lens[s] = 0
    for _ in range(400):
        s = int(rng.integers(0, 40))
        n = int(rng.integers(1, 20))
        pool.prepare_write(s, lens[s], n)
        lens[s] += n
        for t, ln in lens.items():
            waste = len(pool.table(t)) * g["block_size"] - ln
            assert 0 <= waste <= g["max_wasted_slots_per_sequence"], "waste bound broken"


def check_fifo_free_list(bp):
    pool = bp.BlockPool(4, 16, free_order=[3, 1, 0, 2])
    a = pool.add_sequence(); b = pool.add_sequence()
    pool.prepare_write(a, 0, 16)                        # 3
    pool.prepare_write(b, 0, 16)                        # 1
    pool.free_sequence(a)                               # 3 to tail: [0, 2, 3]
    c = pool.add_sequence()
    pool.prepare_write(c, 0, 48)
    assert pool.table(c) == [0, 2, 3]
