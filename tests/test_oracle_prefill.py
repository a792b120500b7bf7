"""Pins of the paged prefill oracle (oracle/paged_prefill.py): its relation to decode,
PyTorch's scaled_dot_product_attention with a causal mask, pure-Python brute force, chunk
consistency; and planted mistakes in copies of it that the pins must catch."""

import os
import sys
import types

import numpy as np
import pytest

import oracle_checks as oc
from oracle import brute
from oracle import paged_attention as pa
from oracle import paged_prefill as pp
from workloads import build_case

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def _chunk_case(lens, chunks, hq, hkv, d, kv_dtype, seed):
    """Contexts of `lens` tokens; sequence s queries its last chunks[s] positions."""
    case = build_case("prefill", lens, hq, hkv, d, kv_dtype, seed)
    rng = np.random.default_rng(seed + 1000)
    T = int(sum(chunks))
    x = rng.standard_normal((T, hq, d)).astype(np.float32)
    q = x if kv_dtype == "f32" else oc.bf16_bits(x)
    cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    return case, q, cu


def check_decode_relation(m):
    """One query token per sequence, at its last position: exactly the decode."""
    case = build_case("rel", [1, 15, 16, 17, 40, 100], 8, 2, 32, "bf16", 21)
    cu = np.arange(case.batch + 1, dtype=np.int32)
    o, l = m.paged_prefill(case.q[0], case.k_pool[0], case.v_pool[0], case.block_tables, cu,
                           case.context_lens, case.scale, "bf16")
    wo, wl = pa.paged_decode(case.q[0], case.k_pool[0], case.v_pool[0], case.block_tables,
                             case.context_lens, case.scale, "bf16")
    assert o.tobytes() == wo.tobytes() and l.tobytes() == wl.tobytes()


def check_sdpa_causal(m, kv_dtype="f32"):
    import torch
    import torch.nn.functional as F
    lens, chunks = [7, 33, 50, 64], [7, 12, 1, 64]
    case, q, cu = _chunk_case(lens, chunks, 6, 2, 16, kv_dtype, 22)
    o, l = m.paged_prefill(q, case.k_pool[0], case.v_pool[0], case.block_tables, cu,
                           case.context_lens, case.scale, kv_dtype)
    G = 3
    for s, (n, L) in enumerate(zip(lens, chunks)):
        ids = case.block_tables[s, :-(-n // 16)]
        K = oc._widen(case.k_pool[0][ids], kv_dtype).transpose(1, 0, 2, 3).reshape(2, -1, 16)[:, :n]
        V = oc._widen(case.v_pool[0][ids], kv_dtype).transpose(1, 0, 2, 3).reshape(2, -1, 16)[:, :n]
        Kt = torch.from_numpy(np.ascontiguousarray(K)).repeat_interleave(G, dim=0)
        Vt = torch.from_numpy(np.ascontiguousarray(V)).repeat_interleave(G, dim=0)
        qs = oc._widen(q[cu[s]:cu[s + 1]], kv_dtype).transpose(1, 0, 2)      # [Hq, L, D]
        qt = torch.from_numpy(np.ascontiguousarray(qs))
        allowed = torch.arange(n)[None, :] <= (n - L + torch.arange(L))[:, None]
        ref = F.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=allowed,
                                             scale=float(case.scale))
        scores = (qt @ Kt.transpose(1, 2)) * float(case.scale)
        ref_lse = torch.logsumexp(scores.masked_fill(~allowed, -float("inf")), dim=-1)
        oc._close(o[cu[s]:cu[s + 1]], ref.numpy().transpose(1, 0, 2), 1e-12, "sdpa out")
        oc._close(l[cu[s]:cu[s + 1]], ref_lse.numpy().T, 1e-12, "sdpa lse")


def check_brute_force(m):
    lens, chunks = [5, 18, 33], [5, 3, 17]
    case, q, cu = _chunk_case(lens, chunks, 4, 2, 2, "f32", 23)
    o, l = m.paged_prefill(q, case.k_pool[0], case.v_pool[0], case.block_tables, cu,
                           case.context_lens, case.scale, "f32")
    kp = case.k_pool[0].astype(np.float64).tolist()
    vp = case.v_pool[0].astype(np.float64).tolist()
    scale = float(np.float32(case.scale))
    for s, (n, L) in enumerate(zip(lens, chunks)):
        row = case.block_tables[s].tolist()
        for i in range(L):
            for h in range(4):
                qh = q[cu[s] + i, h].astype(np.float64).tolist()
                bo, bl = brute.decode_one(qh, kp, vp, row, n - L + i + 1, h // 2, scale)
                oc._close(o[cu[s] + i, h], bo, 1e-12, "brute out")
                oc._close(l[cu[s] + i, h], bl, 1e-12, "brute lse")


def check_chunk_consistency(m):
    """The last c queries of a full prefill equal a prefill of just that chunk."""
    lens = [48, 70]
    case, q, cu = _chunk_case(lens, lens, 8, 4, 16, "bf16", 24)
    full = m.paged_prefill(q, case.k_pool[0], case.v_pool[0], case.block_tables, cu,
                           case.context_lens, case.scale, "bf16")
    tail = [9, 33]
    rows = np.concatenate([np.arange(cu[s + 1] - c, cu[s + 1]) for s, c in enumerate(tail)])
    cu2 = np.concatenate([[0], np.cumsum(tail)]).astype(np.int32)
    part = m.paged_prefill(q[rows], case.k_pool[0], case.v_pool[0], case.block_tables, cu2,
                           case.context_lens, case.scale, "bf16")
    assert part[0].tobytes() == full[0][rows].tobytes()
    assert part[1].tobytes() == full[1][rows].tobytes()


def check_rejects_chunk_outside_context(m):
    case = build_case("bad", [4], 2, 2, 8, "f32", 25)
    q = np.zeros((5, 2, 8), np.float32)
    with pytest.raises(ValueError):
        m.paged_prefill(q, case.k_pool[0], case.v_pool[0], case.block_tables,
                        np.array([0, 5], np.int32), case.context_lens, case.scale, "f32")


CHECKS = [check_decode_relation, check_sdpa_causal, lambda m: check_sdpa_causal(m, "bf16"),
          check_brute_force, check_chunk_consistency, check_rejects_chunk_outside_context]


@pytest.mark.parametrize("i", range(len(CHECKS)))
def test_prefill_oracle_pin(i):
    CHECKS[i](pp)


def _mutant(old, new):
    src = open(os.path.join(ORACLE_DIR, "paged_prefill.py")).read()
    assert old in src, f"mutation anchor not found: {old!r}"
    name = "oracle.mutant_paged_prefill"
    mod = types.ModuleType(name)
    mod.__package__ = "oracle"
    sys.modules[name] = mod
    try:
        exec(compile(src.replace(old, new, 1), "paged_prefill.py", "exec"), mod.__dict__)
    finally:
        del sys.modules[name]
    return mod


MUTANTS = {
    "causal excludes self": ("K[kvh, :pos + 1], V[kvh, :pos + 1]", "K[kvh, :pos], V[kvh, :pos]"),
    "causal sees the next token": ("K[kvh, :pos + 1], V[kvh, :pos + 1]",
                                   "K[kvh, :pos + 2], V[kvh, :pos + 2]"),
    "positions from the chunk start": ("pos = n - L + i", "pos = i"),
    "whole context for every query": ("K[kvh, :pos + 1], V[kvh, :pos + 1]", "K[kvh], V[kvh]"),
    "wrong query row": ("qw[r0 + i, hs]", "qw[i, hs]"),
    "gqa head mapping": ("hs = slice(kvh * G, (kvh + 1) * G)", "hs = slice(kvh, kvh + G)"),
    "rows written reversed": ("out[r0 + i, hs] = o", "out[r1 - 1 - i, hs] = o"),
}


def _caught(mod):
    for chk in CHECKS:
        try:
            with np.errstate(all="ignore"):
                chk(mod)
        except Exception:
            return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_prefill_mutant_is_caught(name):
    assert _caught(_mutant(*MUTANTS[name])), f"{name} survived"
