"""numpy / float64 oracle of paged (chunked) prefill attention (test infrastructure only).

A sequence's new chunk of query tokens attends causally over its paged context (spindle,
"Why write the forward pass" and "Two bugs worth recording": the prompt is processed by
the same forward pass over the block cache, with explicit lengths).  Reading where the
pages are silent, matching the decode path's: the chunk's K/V are appended first, so the
context of sequence s has context_lens[s] tokens including the chunk, and its q_len
query tokens are the last q_len positions of that context.  Query i of the chunk sits
at position n - q_len + i and attends to tokens [0, n - q_len + i].

Layout: q [T, Hq, D] (cache dtype), sequence s owning rows cu_q[s] .. cu_q[s+1] - 1;
caches and block tables as in paged_attention.  Returns out float64 [T, Hq, D] and lse
float64 [T, Hq] (natural log).
"""

from __future__ import annotations

import numpy as np

from .paged_attention import _attend, gather_sequence, widen


def paged_prefill(q, k_pool, v_pool, block_tables, cu_q, context_lens, scale, kv_dtype,
                  block_size: int = 16):
    T, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    scale = float(np.float32(scale))
    out = np.zeros((T, Hq, D))
    lse = np.full((T, Hq), -np.inf)
    qw = widen(q, kv_dtype)
    B = len(context_lens)
    if len(cu_q) != B + 1 or int(cu_q[0]) != 0 or int(cu_q[B]) != T:
        raise ValueError("cu_q must run from 0 to T over batch + 1 entries")
    for s in range(B):
        r0, r1 = int(cu_q[s]), int(cu_q[s + 1])
        L = r1 - r0
        n = int(context_lens[s])
        if L < 0 or L > n:
            raise ValueError("a chunk must lie inside its context")
        if L == 0:
            continue
        K = widen(gather_sequence(k_pool, block_tables[s], n, block_size), kv_dtype)
        V = widen(gather_sequence(v_pool, block_tables[s], n, block_size), kv_dtype)
        for i in range(L):
            pos = n - L + i
            for kvh in range(Hkv):
                hs = slice(kvh * G, (kvh + 1) * G)
                o, l = _attend(qw[r0 + i, hs], K[kvh, :pos + 1], V[kvh, :pos + 1], scale)
                out[r0 + i, hs] = o
                lse[r0 + i, hs] = l
    return out, lse
