"""numpy / float64 oracle of the paged decode path (test infrastructure only).

Data layout (one layer):
  k_pool, v_pool : [num_blocks, num_kv_heads, block_size, head_dim]
                   float32, or uint16 holding bfloat16 bits
  block_tables   : int32 [batch, W]; row s lists sequence s's physical blocks
                   in logical order (spindle, "Paging": block table -> pool)
  context_lens   : int32 [batch]; the explicit number of tokens to attend
                   (spindle, "Two bugs worth recording": gather takes an
                   explicit length; nothing is inferred)
  q              : [batch, num_q_heads, head_dim], same dtype as the pool

Query head h reads KV head h // G with G = num_q_heads / num_kv_heads
(contiguous grouping; the pages are silent on GQA).

All arithmetic is float64 on the exact stored input bits.
"""

from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def widen(x: np.ndarray, kv_dtype: str) -> np.ndarray:
    """Exact float64 values of stored float32 values or bfloat16 bit patterns."""
    if kv_dtype == "f32":
        return np.asarray(x, np.float32).astype(np.float64)
    if kv_dtype == "bf16":
        bits = np.asarray(x, np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(kv_dtype)


def gather_sequence(pool: np.ndarray, table_row: np.ndarray, n: int, block_size: int = 16):
    """Contiguous [Hkv, n, D] copy (same bits, same dtype) of a sequence's first n tokens.

    Logical token t sits in physical block table_row[t // block_size] at slot
    t % block_size (spindle, "Paging").
    """
    num_blocks = pool.shape[0]
    nb = -(-n // block_size)
    ids = np.asarray(table_row[:nb], np.int64)
    if nb and (ids.min() < 0 or ids.max() >= num_blocks):
        raise IndexError("block id out of range")
    blocks = pool[ids]                                  # [nb, Hkv, bs, D]
    seq = blocks.transpose(1, 0, 2, 3).reshape(pool.shape[1], nb * block_size, pool.shape[3])
    return seq[:, :n]


def _attend(qg: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Naive softmax attention of G query rows against n keys, float64.

    qg [G, D], K [n, D], V [n, D] -> (out [G, D], lse [G]); lse is the natural
    log of sum_t exp(score_t).
    """
    s = (qg @ K.T) * scale                               # [G, n]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    out = (e @ V) / l
    lse = (m + np.log(l))[:, 0]
    return out, lse


def paged_decode(q, k_pool, v_pool, block_tables, context_lens, scale, kv_dtype,
                 block_size: int = 16):
    """Single-token decode attention over the block-paged cache.

    Returns (out float64 [B, Hq, D], lse float64 [B, Hq]).  A sequence with
    context length 0 gets out = 0 and lse = -inf.
    """
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    scale = float(np.float32(scale))
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), NEG_INF)
    qw = widen(q, kv_dtype)
    for s in range(B):
        n = int(context_lens[s])
        if n == 0:
            continue
        K = widen(gather_sequence(k_pool, block_tables[s], n, block_size), kv_dtype)
        V = widen(gather_sequence(v_pool, block_tables[s], n, block_size), kv_dtype)
        for kvh in range(Hkv):
            hs = slice(kvh * G, (kvh + 1) * G)
            out[s, hs], lse[s, hs] = _attend(qw[s, hs], K[kvh], V[kvh], scale)
    return out, lse


def contiguous_decode(q, keys, values, scale, kv_dtype):
    """Decode attention over per-sequence contiguous K/V (no paging at all).

    keys[s], values[s]: [Hkv, n_s, D] in the stored dtype.  Written
    independently of ``paged_decode`` (softmax weights from a log-sum-exp,
    per query head) so that the two can pin each other.
    """
    B, Hq, D = q.shape
    scale = float(np.float32(scale))
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), NEG_INF)
    qw = widen(q, kv_dtype)
    for s in range(B):
        K = widen(keys[s], kv_dtype)
        V = widen(values[s], kv_dtype)
        Hkv, n, _ = K.shape
        if n == 0:
            continue
        per_kv = Hq // Hkv
        for h in range(Hq):
            kvh = h // per_kv
            logits = scale * np.einsum("td,d->t", K[kvh], qw[s, h])
            z = np.logaddexp.reduce(logits)
            w = np.exp(logits - z)
            out[s, h] = np.einsum("t,td->d", w, V[kvh])
            lse[s, h] = z
    return out, lse


def decode_partitions(q, k_pool, v_pool, block_tables, context_lens, scale, kv_dtype,
                      partition_size: int, block_size: int = 16):
    """Flash-decoding first pass: attention restricted to each KV partition.

    Partition p of sequence s covers tokens [p*P, min((p+1)*P, n)).  Returns
    (part_out [B, Hq, NP, D], part_lse [B, Hq, NP]) with NP = max_s ceil(n_s/P)
    (at least 1); partitions past a sequence's end hold out = 0, lse = -inf.
    """
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    P = int(partition_size)
    if P <= 0 or P % block_size:
        raise ValueError("partition_size must be a positive multiple of the block size")
    scale = float(np.float32(scale))
    NP = max(1, max((-(-int(n) // P) for n in context_lens), default=1))
    part_out = np.zeros((B, Hq, NP, D))
    part_lse = np.full((B, Hq, NP), NEG_INF)
    qw = widen(q, kv_dtype)
    for s in range(B):
        n = int(context_lens[s])
        if n == 0:
            continue
        K = widen(gather_sequence(k_pool, block_tables[s], n, block_size), kv_dtype)
        V = widen(gather_sequence(v_pool, block_tables[s], n, block_size), kv_dtype)
        for p in range(-(-n // P)):
            ts = slice(p * P, min((p + 1) * P, n))
            for kvh in range(Hkv):
                hs = slice(kvh * G, (kvh + 1) * G)
                o, l = _attend(qw[s, hs], K[kvh, ts], V[kvh, ts], scale)
                part_out[s, hs, p] = o
                part_lse[s, hs, p] = l
    return part_out, part_lse


def combine_partitions(part_out, part_lse):
    """Second pass: merge per-partition results by their log-sum-exp.

    out = sum_p exp(lse_p - M) O_p / sum_p exp(lse_p - M), lse = M + ln sum_p
    exp(lse_p - M), M = max_p lse_p, over partitions with lse_p > -inf.  All
    partitions empty -> out = 0, lse = -inf.
    """
    part_out = np.asarray(part_out, np.float64)
    part_lse = np.asarray(part_lse, np.float64)
    B, Hq, NP, D = part_out.shape
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), NEG_INF)
    for s in range(B):
        for h in range(Hq):
            lv = part_lse[s, h]
            live = lv > NEG_INF
            if not live.any():
                continue
            M = lv[live].max()
            w = np.exp(lv[live] - M)
            out[s, h] = (w[:, None] * part_out[s, h, live]).sum(axis=0) / w.sum()
            lse[s, h] = M + np.log(w.sum())
    return out, lse


def kv_append(k_pool, v_pool, k_new, v_new, block_tables, start_pos, cu_new_tokens,
              block_size: int = 16, inplace: bool = False):
    """Write new tokens' K/V into their blocks at an explicit start position.

    Token i of sequence s (global row cu_new_tokens[s] + i of k_new/v_new,
    [T, Hkv, D]) lands at logical position start_pos[s] + i, i.e. physical
    block block_tables[s][pos // bs], slot pos % bs, for every KV head.  A raw
    bit copy; returns new pools and leaves the inputs untouched, or writes into
    the given pools when inplace=True (long replays).
    """
    k_out = k_pool if inplace else k_pool.copy()
    v_out = v_pool if inplace else v_pool.copy()
    W = block_tables.shape[1]
    NB = k_pool.shape[0]
    B = len(start_pos)
    for s in range(B):
        for i in range(int(cu_new_tokens[s + 1]) - int(cu_new_tokens[s])):
            pos = int(start_pos[s]) + i
            if pos < 0 or pos >= W * block_size:
                raise IndexError("append position outside the block table")
            blk = int(block_tables[s, pos // block_size])
            if blk < 0 or blk >= NB:
                raise IndexError("block id out of range")
            row = int(cu_new_tokens[s]) + i
            k_out[blk, :, pos % block_size, :] = k_new[row]
            v_out[blk, :, pos % block_size, :] = v_new[row]
    return k_out, v_out


def copy_blocks(k_pool, v_pool, src, dst):
    """Copy-on-write block copy: pool[dst[i]] = pool[src[i]] bitwise, in list order."""
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    for a, b in zip(src, dst):
        k_out[int(b)] = k_out[int(a)]
        v_out[int(b)] = v_out[int(a)]
    return k_out, v_out
