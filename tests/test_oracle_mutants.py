"""Plant plausible mistakes in copies of the oracle (on the CPU) and require the
pins to catch every one: evidence that the pins constrain the oracle's
arithmetic and indexing, not just that it runs."""

import os
import types
import warnings

import numpy as np
import pytest

import oracle_checks as oc

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def _mutant(module_file, old, new, count=1):
    src = open(os.path.join(ORACLE_DIR, module_file)).read()
    assert src.count(old) >= count, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("mutant_" + module_file[:-3])
    mod.__dict__["__name__"] = mod.__name__
    exec(compile(src.replace(old, new, count), module_file, "exec"), mod.__dict__)
    return mod


PA_CHECKS = [
    oc.check_gather_roundtrip,
    lambda m: oc.check_gather_roundtrip(m, "bf16"),
    oc.check_paged_vs_contiguous,
    oc.check_closed_forms,
    oc.check_library_sdpa,
    oc.check_permutation_invariance,
    oc.check_batched_equals_alone,
    oc.check_forks_identical,
    oc.check_append,
    oc.check_copy_blocks,
    oc.check_split_identity,
    lambda m: oc.check_split_identity(m, q_scale=400.0),
    oc.check_brute_force,
]

BP_CHECKS = [oc.check_cow_golden, oc.check_cow_write, oc.check_waste_bound,
             oc.check_fifo_free_list]

PA_MUTANTS = {
    "dropped scale": ("s = (qg @ K.T) * scale", "s = (qg @ K.T)"),
    "wrong sign in exp": ("e = np.exp(s - m)", "e = np.exp(m - s)"),
    "lse drops max": ("lse = (m + np.log(l))[:, 0]", "lse = (np.log(l))[:, 0]"),
    "no normalisation": ("out = (e @ V) / l", "out = (e @ V)"),
    "gqa head mapping": ("            hs = slice(kvh * G, (kvh + 1) * G)\n            out[s, hs]",
                         "            hs = slice(kvh, kvh + G)\n            out[s, hs]"),
    "gather without transpose": ("blocks.transpose(1, 0, 2, 3)", "blocks.transpose(0, 1, 2, 3)"),
    "gather reversed blocks": ("ids = np.asarray(table_row[:nb], np.int64)",
                               "ids = np.asarray(table_row[:nb][::-1], np.int64)"),
    "gather drops tail": ("return seq[:, :n]", "return seq[:, :max(n - 1, 1)]"),
    "decode one short": ("n = int(context_lens[s])\n        if n == 0:\n            continue\n        K = widen",
                         "n = max(int(context_lens[s]) - 1, 1)\n        if n == 0:\n            continue\n        K = widen"),
    "bf16 widened wrong": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "append off by one": ("pos = int(start_pos[s]) + i", "pos = int(start_pos[s]) + i + 1"),
    "append wrong slot": ("k_out[blk, :, pos % block_size, :] = k_new[row]",
                          "k_out[blk, :, (pos + 1) % block_size, :] = k_new[row]"),
    "append wrong row": ("row = int(cu_new_tokens[s]) + i", "row = int(cu_new_tokens[s])"),
    "copy reversed": ("k_out[int(b)] = k_out[int(a)]", "k_out[int(a)] = k_out[int(b)]"),
    "partition drops last token": ("ts = slice(p * P, min((p + 1) * P, n))",
                                   "ts = slice(p * P, min((p + 1) * P, n) - 1)"),
    "combine without max shift": ("w = np.exp(lv[live] - M)", "w = np.exp(lv[live])"),
    "combine lse drops max": ("lse[s, h] = M + np.log(w.sum())", "lse[s, h] = np.log(w.sum())"),
    "combine unweighted": ("out[s, h] = (w[:, None] * part_out[s, h, live]).sum(axis=0) / w.sum()",
                           "out[s, h] = part_out[s, h, live].mean(axis=0)"),
}

BP_MUTANTS = {
    "lifo free list": ("self.free.append(b)", "self.free.appendleft(b)"),
    "frees shared block": ("if self.refcount[b] == 0:", "if self.refcount[b] <= 1:"),
    "no copy on write": ("elif self.refcount[table[j]] > 1:", "elif self.refcount[table[j]] > 2:"),
    "fork forgets refcount": ("            self.refcount[b] += 1\n", "            pass\n"),
    "not atomic": ("if need > len(self.free):", "if False:"),
}


def _caught(checks, mod):
    for chk in checks:
        try:
            with warnings.catch_warnings():
                warnings.simplefilter("ignore")
                with np.errstate(all="ignore"):
                    chk(mod)
        except Exception:  # AssertionError, or the mutant crashing outright
            return True
    return False


def test_unmutated_oracle_passes_every_check():
    mod = _mutant("paged_attention.py", "", "", 0)
    assert not _caught(PA_CHECKS, mod)
    mod = _mutant("block_pool.py", "", "", 0)
    assert not _caught(BP_CHECKS, mod)


@pytest.mark.parametrize("name", sorted(PA_MUTANTS))
def test_attention_mutant_is_caught(name):
    old, new = PA_MUTANTS[name]
    assert _caught(PA_CHECKS, _mutant("paged_attention.py", old, new)), f"{name} survived"


@pytest.mark.parametrize("name", sorted(BP_MUTANTS))
def test_block_pool_mutant_is_caught(name):
    old, new = BP_MUTANTS[name]
    assert _caught(BP_CHECKS, _mutant("block_pool.py", old, new)), f"{name} survived"
