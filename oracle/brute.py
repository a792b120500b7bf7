"""Pure-Python brute force of the same definitions (test infrastructure only).

Explicit loops over nested lists with ``math.exp``, ``math.log`` and
``math.fsum``; float64 throughout.  Meant for tiny inputs (a few blocks, a
handful of dimensions) to pin the numpy oracle.  Inputs are plain float64
nested lists (already widened) plus integer tables.
"""

from __future__ import annotations

import math


def token_location(table_row, t, block_size=16):
    """Physical (block id, slot) of logical token t."""
    return table_row[t // block_size], t % block_size


def decode_one(q_head, pool_k, pool_v, table_row, n, kv_head, scale, block_size=16):
    """out[D], lse for one query head of one sequence.

    pool_k[b][h][slot][d] as nested lists of floats.
    """
    if n == 0:
        return [0.0] * len(q_head), -math.inf
    scores = []
    for t in range(n):
        b, slot = token_location(table_row, t, block_size)
        k = pool_k[b][kv_head][slot]
        scores.append(scale * math.fsum(q_head[d] * k[d] for d in range(len(q_head))))
    m = max(scores)
    weights = [math.exp(x - m) for x in scores]
    total = math.fsum(weights)
    out = []
    for d in range(len(q_head)):
        acc = []
        for t in range(n):
            b, slot = token_location(table_row, t, block_size)
            acc.append(weights[t] * pool_v[b][kv_head][slot][d])
        out.append(math.fsum(acc) / total)
    return out, m + math.log(total)


def decode(q, pool_k, pool_v, tables, ctx, scale, block_size=16):
    """q[s][h][d] -> (out[s][h][d], lse[s][h])."""
    Hq = len(q[0])
    Hkv = len(pool_k[0])
    G = Hq // Hkv
    out, lse = [], []
    for s in range(len(q)):
        orow, lrow = [], []
        for h in range(Hq):
            o, l = decode_one(q[s][h], pool_k, pool_v, tables[s], ctx[s], h // G, scale,
                              block_size)
            orow.append(o)
            lrow.append(l)
        out.append(orow)
        lse.append(lrow)
    return out, lse


def combine(parts_out, parts_lse):
    """Merge one head's partitions: lists of out vectors and lse scalars."""
    live = [i for i, l in enumerate(parts_lse) if l != -math.inf]
    D = len(parts_out[0])
    if not live:
        return [0.0] * D, -math.inf
    M = max(parts_lse[i] for i in live)
    w = {i: math.exp(parts_lse[i] - M) for i in live}
    tot = math.fsum(w.values())
    out = [math.fsum(w[i] * parts_out[i][d] for i in live) / tot for d in range(D)]
    return out, M + math.log(tot)


def append(pool, new_rows, table_row, start, block_size=16):
    """Write rows new_rows[i] (each [Hkv][D]) at positions start + i; in place."""
    for i, row in enumerate(new_rows):
        b, slot = token_location(table_row, start + i, block_size)
        for h in range(len(row)):
            pool[b][h][slot] = list(row[h])
    return pool
