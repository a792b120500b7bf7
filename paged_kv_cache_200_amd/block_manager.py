"""Python handle over the native block manager (pkv_bm_* in libpkv.so).

Host bookkeeping of the paged pool: FIFO free list, per-sequence block tables,
reference counts, fork and copy-on-write (spindle, "Paging").  The copies that
a write requires are returned as (src, dst) block-id pairs; ``apply_copies``
moves the data on the GPU with the library's block-copy kernel.
"""

from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _lib, ops


class OutOfBlocks(RuntimeError):
    """The pool has fewer free blocks than the write needs (nothing was changed)."""


def _i32p(arr: np.ndarray):
    return arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int = 16, free_order=None):
        self._lib = _lib.lib()
        self._h = ctypes.c_void_p()
        order = None
        if free_order is not None:
            order = np.ascontiguousarray(np.asarray(free_order, np.int32))
        _lib.call("pkv_bm_create", int(num_blocks), int(block_size),
                  None if order is None else order.ctypes.data, ctypes.byref(self._h))
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.pkv_bm_destroy(h)
            self._h = None

    def add_sequence(self) -> int:
        out = ctypes.c_int32()
        _lib.call("pkv_bm_add_sequence", self._h, ctypes.byref(out))
        return out.value

    def prepare_write(self, seq: int, start: int, n: int):
        """Make positions [start, start+n) of seq writable; returns [(src, dst), ...] copies."""
        cap = n // self.block_size + 2
        src = np.zeros(cap, np.int32)
        dst = np.zeros(cap, np.int32)
        cnt = ctypes.c_int32()
        st = self._lib.pkv_bm_prepare_write(self._h, int(seq), int(start), int(n), _i32p(src),
                                            _i32p(dst), cap, ctypes.byref(cnt))
        if st == _lib.PKV_ERR_OUT_OF_BLOCKS:
            raise OutOfBlocks("block pool exhausted")
        _lib.check("pkv_bm_prepare_write", st)
        return [(int(a), int(b)) for a, b in zip(src[:cnt.value], dst[:cnt.value])]

    def prepare_step(self, seqs, starts, counts, width: int, pad_id: int = 0,
                     tables_out: np.ndarray | None = None):
        """One step's writes and tables in one native call: prepare_write(seqs[r], starts[r],
        counts[r]) for every r in order, then the dense int32 [len(seqs), width] tables
        (into tables_out when given).  Returns (tables, [(src, dst), ...] copies).  On an
        exhausted pool raises OutOfBlocks; the writes before the failing sequence stay done."""
        s = np.ascontiguousarray(np.asarray(seqs, np.int32))
        st_ = np.ascontiguousarray(np.asarray(starts, np.int32))
        ct = np.ascontiguousarray(np.asarray(counts, np.int32))
        n = len(s)
        out = tables_out if tables_out is not None else np.empty((n, width), np.int32)
        if out.shape != (n, width) or out.dtype != np.int32 or not out.flags.c_contiguous:
            raise ValueError("tables_out must be a contiguous int32 [len(seqs), width] array")
        cap = int(ct.sum()) // self.block_size + 2 * n + 1
        src = np.zeros(cap, np.int32)
        dst = np.zeros(cap, np.int32)
        cnt, done = ctypes.c_int32(), ctypes.c_int32()
        st = self._lib.pkv_bm_prepare_step(self._h, _i32p(s), _i32p(st_), _i32p(ct), n,
                                           _i32p(out), int(width), int(pad_id), _i32p(src),
                                           _i32p(dst), cap, ctypes.byref(cnt),
                                           ctypes.byref(done))
        if st == _lib.PKV_ERR_OUT_OF_BLOCKS:
            raise OutOfBlocks(f"block pool exhausted at sequence {s[done.value]}")
        _lib.check("pkv_bm_prepare_step", st)
        return out, [(int(a), int(b)) for a, b in zip(src[:cnt.value], dst[:cnt.value])]

    def fork(self, parent: int) -> int:
        out = ctypes.c_int32()
        _lib.call("pkv_bm_fork", self._h, int(parent), ctypes.byref(out))
        return out.value

    def free_sequence(self, seq: int) -> None:
        _lib.call("pkv_bm_free_sequence", self._h, int(seq))

    def num_blocks_of(self, seq: int) -> int:
        out = ctypes.c_int32()
        _lib.call("pkv_bm_num_blocks_of", self._h, int(seq), ctypes.byref(out))
        return out.value

    def table(self, seq: int):
        n = self.num_blocks_of(seq)
        return self.tables([seq], max(n, 1), pad_id=-1)[0, :n].tolist()

    def tables(self, seqs, width: int, pad_id: int = 0) -> np.ndarray:
        """Dense int32 [len(seqs), width] tables, padded with pad_id."""
        s = np.ascontiguousarray(np.asarray(seqs, np.int32))
        out = np.empty((len(s), width), np.int32)
        _lib.call("pkv_bm_fill_tables", self._h, _i32p(s), len(s), _i32p(out), int(width),
                  int(pad_id))
        return out

    def refcount(self, block: int) -> int:
        out = ctypes.c_int32()
        _lib.call("pkv_bm_refcount", self._h, int(block), ctypes.byref(out))
        return out.value

    def num_free(self) -> int:
        out = ctypes.c_int32()
        _lib.call("pkv_bm_num_free", self._h, ctypes.byref(out))
        return out.value

    def free_list(self):
        n = self.num_free()
        ids = np.zeros(max(n, 1), np.int32)
        cnt = ctypes.c_int32()
        _lib.call("pkv_bm_free_list", self._h, _i32p(ids), len(ids), ctypes.byref(cnt))
        return ids[:cnt.value].tolist()

    @staticmethod
    def apply_copies(copies, k_cache: torch.Tensor, v_cache: torch.Tensor, stream=None) -> None:
        """Run the block copies on the GPU (caches [NB, ...] or stacked layers [L, NB, ...])."""
        if not copies:
            return
        pairs = torch.tensor(copies, dtype=torch.int32)
        src = pairs[:, 0].contiguous().to(k_cache.device)
        dst = pairs[:, 1].contiguous().to(k_cache.device)
        ops.copy_blocks(k_cache, v_cache, src, dst, stream=stream)
