"""Helpers shared by the GPU tests: move seeded cases to the device, run the
library, compare with the oracle under the stated tolerances."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle.paged_attention as pa

# max-abs tolerances on out and lse: fp32 caches / bf16 caches with fp32 accumulation
TOL = {"f32": 2e-3, "bf16": 1e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray) -> torch.Tensor:
    """Host array -> device tensor with the same bits (bf16 bit patterns as int16)."""
    if x.dtype == np.uint16:
        x = x.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host_bits(t: torch.Tensor, kv_dtype: str) -> np.ndarray:
    a = t.cpu().numpy()
    return a.view(np.uint16) if kv_dtype == "bf16" else a


class DeviceCase:
    def __init__(self, case, layer=0):
        self.case = case
        self.q = dev(case.q[layer])
        self.k = dev(case.k_pool[layer])
        self.v = dev(case.v_pool[layer])
        self.tables = dev(case.block_tables)
        self.ctx = dev(case.context_lens)
        self.max_ctx = int(case.context_lens.max()) if case.batch else 0


def run_decode(dc: DeviceCase, partition_size=0, max_ctx=None, q=None):
    from paged_kv_cache_200_amd import ops
    out, lse = ops.paged_decode(dc.q if q is None else q, dc.k, dc.v, dc.tables, dc.ctx,
                                dc.max_ctx if max_ctx is None else max_ctx,
                                scale=float(dc.case.scale), partition_size=partition_size)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def oracle_decode(case, layer=0, q=None):
    return pa.paged_decode(case.q[layer] if q is None else q, case.k_pool[layer],
                           case.v_pool[layer], case.block_tables, case.context_lens, case.scale,
                           case.kv_dtype)


def max_abs_err(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin), "finite/infinite pattern differs"
    assert np.array_equal(got[~fin], want[~fin]), "infinite entries differ"
    return float(np.max(np.abs(got[fin] - want[fin]))) if fin.any() else 0.0


def assert_parity(got, want, kv_dtype, what=""):
    (go, gl), (wo, wl) = got, want
    eo = max_abs_err(go, wo)
    el = max_abs_err(gl, wl)
    say(f"  {what}: max|out err| {eo:.3e}  max|lse err| {el:.3e}  (tol {TOL[kv_dtype]})")
    assert eo <= TOL[kv_dtype], f"{what}: out error {eo}"
    assert el <= TOL[kv_dtype], f"{what}: lse error {el}"
    return eo, el


def assert_no_device_error():
    from paged_kv_cache_200_amd import ops
    flags = ops.device_error()
    assert flags == 0, f"device error bits set: {ops.describe_device_error(flags)}"
