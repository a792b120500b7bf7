"""One-hot gather probes (test infrastructure; the GPU path never imports this).

A probe turns attention into a pure indexing question whose answer is one stored V row,
exactly.  Every query row is a one-hot vector e_j (value 1) with softmax scale 1, so
its score against a key is that key's value in dimension j.  Keys a row may attend are set
to 0 in the probed dimensions, except "hot" keys holding LEVEL * k for small integers k.
The key of the largest level a row can see scores at least LEVEL above every other, so
its softmax weight is exp(0) = 1 and every other weight is below e^-160: that underflows
to 0 in float32 (the kernels' exp2 of a value below -230), and in the float64 oracle it
perturbs the result by ~1e-70 relative, which rounding to float32 cannot show.  The exact
result is therefore the hot key's V row, the same float32 values on both sides (a stored
-0.0 may come back as +0.0: sums start from +0, and the oracle's sign there is that of its
tiny remainder).  A row whose
gather reaches a wrong block, slot or KV head, reads past its length, or misses its hot key
returns some other row, a mean of rows, or NaN (unused slots hold NaN).

Levels 160 k are exact in bfloat16 for k <= 51 (160 k = 32 * 5k, 5k < 256).

Where the hot keys go:
  decode  : one level-1 hot key per (sequence, KV head, dimension).  Over a sequence's
            Hkv * D probes the hot blocks are consecutive (kv head fastest), from a seeded
            offset, so every block position is hit when Hkv * D >= the block count
            (``phase`` shifts the window for longer sequences); dimension 0 of every KV
            head takes the newest token (the one a decode step appends).  Query head
            h = kh * G + g reads dimension (r * G + g) mod D in round r.
  forks   : a group's shared prefix gets one level-1 key per (KV head, dimension); each
            member with private tokens gets a level-2 key in its private range in odd
            dimensions, which it must prefer; members without private tokens, and even
            dimensions, answer the prefix key.
  prefill : query row (token i, head g) of a chunk reads dimension (i * G + g) mod D; the
            rows sharing a dimension have increasing causal limits and get levels 1, 2, ...
            in that order, each level's hot key lying after the previous row's limit and
            at or before its own, so a row sees its own level and lower ones only; a row
            that sees past its causal limit picks a higher level's key instead.
"""

from __future__ import annotations

import numpy as np

import oracle.paged_attention as pa

LEVEL = 160.0
BS = 16


def stored(value: float, kv_dtype: str):
    """The stored bits of a float32 value (bfloat16: exact values only)."""
    x = np.float32(value)
    if kv_dtype == "f32":
        return x
    bits = np.array([x], np.float32).view(np.uint32)[0]
    assert bits & 0xFFFF == 0, f"{value} is not exact in bfloat16"
    return np.uint16(bits >> 16)


def _zero(kv_dtype):
    return np.float32(0.0) if kv_dtype == "f32" else np.uint16(0)


def clear_live_keys(k_pool, tables, lens, kv_dtype, skip_last=False):
    """K of every token a sequence attends := 0 in every dimension (unused slots keep their
    poison).  skip_last leaves each sequence's newest token alone."""
    z = _zero(kv_dtype)
    for s, n in enumerate(np.asarray(lens).tolist()):
        m = n - 1 if (skip_last and n > 0) else n
        full, r = m // BS, m % BS
        if full:
            k_pool[tables[s, :full]] = z
        if r:
            k_pool[tables[s, full], :, :r, :] = z


def _put(k_pool, tables, s, t, kh, j, level, kv_dtype):
    """K of logical token(s) t of sequence s, KV head(s) kh, dimension(s) j := LEVEL*level."""
    t = np.asarray(t)
    blk = tables[s, t // BS]
    k_pool[blk, kh, t % BS, j] = stored(LEVEL * level, kv_dtype)


def decode_probe(case, layer=0, phase=0, seed=0):
    """Rewrite case.k_pool[layer] in place into a decode probe; returns hot int64
    [B, Hkv, D]: the logical token each (sequence, KV head, dimension) answers (-1 for an
    empty sequence).  The case must not share blocks between sequences."""
    assert not case.shared_blocks, "use fork_probe for copy-on-write cases"
    kp = case.k_pool[layer]
    B, Hkv, D = case.batch, case.num_kv_heads, case.head_dim
    clear_live_keys(kp, case.block_tables, case.context_lens, case.kv_dtype)
    rng = np.random.default_rng(seed)
    hot = np.full((B, Hkv, D), -1, np.int64)
    kh_idx = np.arange(Hkv)[:, None].repeat(D, 1)
    j_idx = np.arange(D)[None, :].repeat(Hkv, 0)
    for s, n in enumerate(case.context_lens.tolist()):
        if n == 0:
            continue
        nblk = -(-n // BS)
        k = j_idx * Hkv + kh_idx
        b = (k + phase * Hkv * D + int(rng.integers(nblk))) % nblk
        valid = np.minimum(BS, n - b * BS)
        t = b * BS + (rng.random(b.shape) * valid).astype(np.int64)
        t[:, 0] = n - 1
        hot[s] = t
        _put(kp, case.block_tables, s, t, kh_idx, j_idx, 1, case.kv_dtype)
    return hot


def fork_probe(case, group_starts, group_shared_blocks, layer=0, seed=0):
    """Probe for a copy-on-write fork case (members of a group consecutive, sharing their
    leading group_shared_blocks blocks); rewrites case.k_pool[layer]; returns hot as
    decode_probe does."""
    kp = case.k_pool[layer]
    B, Hkv, D = case.batch, case.num_kv_heads, case.head_dim
    lens = case.context_lens
    clear_live_keys(kp, case.block_tables, lens, case.kv_dtype)
    rng = np.random.default_rng(seed)
    hot = np.full((B, Hkv, D), -1, np.int64)
    kh_idx = np.arange(Hkv)[:, None].repeat(D, 1)
    j_idx = np.arange(D)[None, :].repeat(Hkv, 0)
    for g in range(len(group_shared_blocks)):
        m0, m1 = int(group_starts[g]), int(group_starts[g + 1])
        members = list(range(m0, m1))
        nmin = min(int(lens[s]) for s in members)
        S = min(int(group_shared_blocks[g]) * BS, nmin)
        if S > 0:
            tp = (rng.random((Hkv, D)) * S).astype(np.int64)
            _put(kp, case.block_tables, m0, tp, kh_idx, j_idx, 1, case.kv_dtype)
        for s in members:
            n = int(lens[s])
            if n == 0:
                continue
            if S > 0:
                hot[s] = tp
            if n > S:
                tq = S + (rng.random((Hkv, D)) * (n - S)).astype(np.int64)
                if S == 0:  # nothing shared: a plain probe in every dimension
                    _put(kp, case.block_tables, s, tq, kh_idx, j_idx, 1, case.kv_dtype)
                    hot[s] = tq
                else:
                    odd = j_idx % 2 == 1
                    _put(kp, case.block_tables, s, tq[odd], kh_idx[odd], j_idx[odd], 2,
                         case.kv_dtype)
                    hot[s][odd] = tq[odd]
    return hot


def decode_rounds(num_q_heads, num_kv_heads, head_dim):
    """Number of decode rounds that probe every dimension of every KV head."""
    G = num_q_heads // num_kv_heads
    return -(-head_dim // G)


def decode_round_q(batch, num_q_heads, num_kv_heads, head_dim, r, kv_dtype):
    """q [B, Hq, D] of round r: head kh * G + g is e_j, j = (r * G + g) mod D; and the
    dimension each head reads, int64 [Hq]."""
    G = num_q_heads // num_kv_heads
    dims = (r * G + np.arange(num_q_heads) % G) % head_dim
    dt = np.float32 if kv_dtype == "f32" else np.uint16
    q = np.zeros((batch, num_q_heads, head_dim), dt)
    q[:, np.arange(num_q_heads), dims] = stored(1.0, kv_dtype)
    return q, dims


def v_rows(v_pool, tables, lens, kv_dtype):
    """Per sequence, the oracle's contiguous gather of V as float32 [Hkv, n, D]."""
    return [pa.widen(pa.gather_sequence(v_pool, tables[s], int(n)), kv_dtype).astype(np.float32)
            for s, n in enumerate(np.asarray(lens).tolist())]


def decode_expected(vseq, hot, num_q_heads, dims):
    """Expected out float32 [B, Hq, D] of a decode round: row (s, h) is V of KV head
    h // G at the hot token of (s, h // G, dims[h]); zeros for empty sequences."""
    B, Hkv, _ = hot.shape
    G = num_q_heads // Hkv
    D = vseq[0].shape[2] if B else 0
    want = np.zeros((B, num_q_heads, D), np.float32)
    for s in range(B):
        if vseq[s].shape[1] == 0:
            continue
        kh = np.arange(num_q_heads) // G
        t = hot[s, kh, dims]
        want[s] = vseq[s][kh, t]
    return want


def check_decode_hot(case, hot, layer=0):
    """The probe's construction, checked on the pool: for every (s, kv head, dim) the hot
    token holds the unique maximum key of the sequence, LEVEL above every other."""
    lv = []
    for s, n in enumerate(case.context_lens.tolist()):
        if n == 0:
            continue
        K = pa.widen(pa.gather_sequence(case.k_pool[layer], case.block_tables[s], n),
                     case.kv_dtype)                      # [Hkv, n, D]
        top = np.argmax(K, axis=1)
        assert np.array_equal(top, hot[s]), f"sequence {s}: argmax differs from the hot map"
        mx = np.take_along_axis(K, top[:, None, :], 1)[:, 0]
        K2 = K.copy()
        np.put_along_axis(K2, top[:, None, :], -np.inf, 1)
        second = K2.max(axis=1) if n > 1 else np.full_like(mx, -np.inf)
        assert np.all(mx - second >= LEVEL), f"sequence {s}: hot key not {LEVEL} above the rest"
        lv.append(mx)
    return lv


def prefill_probe(case, k_new, cu_q, start_pos, layer=0, seed=0):
    """Rewrite a chunked-prefill input into a probe.

    case: pools and tables of the full contexts; k_new [T, Hkv, D]: the chunks' keys,
    appended at start_pos[s] before the prefill (rows cu_q[s] ..), or None when the pool
    already holds the chunks' keys.  The chunk of sequence s is its last q_len tokens, so
    start_pos[s] = n - q_len.  Rewrites the pool's keys (and k_new) in place.  Returns
    (q [T, Hq, D], hot int64 [T, Hq]: the logical token each query row answers)."""
    kp = case.k_pool[layer]
    B, Hq, Hkv, D = case.batch, case.num_q_heads, case.num_kv_heads, case.head_dim
    G = Hq // Hkv
    kvd = case.kv_dtype
    T = int(cu_q[-1])
    dt = np.float32 if kvd == "f32" else np.uint16
    z = _zero(kvd)
    lens = case.context_lens
    prior = np.asarray(start_pos, np.int64)
    clear_live_keys(kp, case.block_tables, lens if k_new is None else prior, kvd)
    if k_new is not None:
        k_new[:] = z
    q = np.zeros((T, Hq, D), dt)
    hot = np.full((T, Hq), -1, np.int64)
    rng = np.random.default_rng(seed)

    def put(s, t, kh, j, level):
        if k_new is not None and t >= prior[s]:
            k_new[int(cu_q[s]) + t - int(prior[s]), kh, j] = stored(LEVEL * level, kvd)
        else:
            _put(kp, case.block_tables, s, t, kh, j, level, kvd)

    for s in range(B):
        r0, r1 = int(cu_q[s]), int(cu_q[s + 1])
        L, n = r1 - r0, int(lens[s])
        assert int(prior[s]) == n - L, "the chunk must be the context's last tokens"
        for kh in range(Hkv):
            last_limit = {}                      # dim -> (level, limit) of its last row
            for i in range(L):
                lim = n - L + i                  # query i attends tokens [0, lim]
                for g in range(G):
                    j = (i * G + g) % D
                    lvl, prev = last_limit.get(j, (0, -1))
                    lo = prev + 1
                    u = rng.random()
                    # boundary and diagonal keys often, anywhere in range otherwise
                    t = lo if u < 0.25 else lim if u < 0.5 else lo + int(rng.integers(lim - lo + 1))
                    put(s, t, kh, j, lvl + 1)
                    last_limit[j] = (lvl + 1, lim)
                    q[r0 + i, kh * G + g, j] = stored(1.0, kvd)
                    hot[r0 + i, kh * G + g] = t
    return q, hot


def prefill_expected(vseq, hot, cu_q, num_q_heads, num_kv_heads):
    """Expected out float32 [T, Hq, D]: V of the row's KV head at its hot token."""
    G = num_q_heads // num_kv_heads
    T = hot.shape[0]
    D = vseq[0].shape[2]
    want = np.zeros((T, num_q_heads, D), np.float32)
    kh = np.arange(num_q_heads) // G
    for s in range(len(cu_q) - 1):
        for r in range(int(cu_q[s]), int(cu_q[s + 1])):
            want[r] = vseq[s][kh, hot[r]]
    return want


def hot_rows(v_pool, tables, lens, hot, kv_dtype):
    """float32 [B, Hkv, D, D]: the V row of every decode probe's hot token, read through
    the oracle's gather (zeros for empty sequences)."""
    B, Hkv, Dj = hot.shape
    D = v_pool.shape[-1]
    rows = np.zeros((B, Hkv, Dj, D), np.float32)
    kh = np.arange(Hkv)[:, None]
    for s, n in enumerate(np.asarray(lens).tolist()):
        if n == 0:
            continue
        V = pa.gather_sequence(v_pool, tables[s], int(n))      # [Hkv, n, D], stored bits
        rows[s] = pa.widen(V[kh, hot[s]], kv_dtype).astype(np.float32)
    return rows


def round_expected(rows, dims, num_q_heads):
    """Expected out float32 [B, Hq, D] of a decode round from hot_rows()."""
    Hkv = rows.shape[1]
    kh = np.arange(num_q_heads) // (num_q_heads // Hkv)
    return np.ascontiguousarray(rows[:, kh, dims])
