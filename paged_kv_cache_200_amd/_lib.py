"""ctypes declarations of libpkv.so (include/pkv.h, include/pkv_block_manager.h,
include/pkv_replay.h).

The library must have been built (``python -m paged_kv_cache_200_amd.build``);
there is no fallback: importing the ops without it raises.  torch is imported
first so that the HIP runtime torch ships is the one libpkv binds to (both
carry the soname libamdhip64.so.7), which makes torch's stream handles valid
arguments.
"""

from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must be loaded before libpkv: shared HIP runtime)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")

PKV_F32 = 0
PKV_BF16 = 1

PKV_OK = 0
PKV_ERR_OUT_OF_BLOCKS = -7
PKV_ERR_SCRATCH = -9
# size of the library's static per-device scratch array (PKV_STATIC_SCRATCH_BYTES)
STATIC_SCRATCH_BYTES = 16 << 20

DEVICE_ERROR_BITS = {
    1: "block id out of range",
    2: "append position outside the block table",
    4: "context length < 0 or beyond the block table",
    8: "context length above max_context_len",
    16: "cu_new_tokens malformed",
    32: "fork groups do not tile the batch",
}

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_pi32 = ctypes.POINTER(ctypes.c_int32)

# name -> (restype, argtypes); the order and names follow the headers.
SIGNATURES = {
    "pkv_version": (ctypes.c_int, []),
    "pkv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pkv_kv_append": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _i32, _i32, _i32,
                                     _i32, _i32, _i32, _i32, _vp]),
    "pkv_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "pkv_decode_partition_size": (_i32, [_i32, _i32, _i32, _i32, _i64]),
    "pkv_decode_engine": (_i32, [_i32, _i32, _i32, _i32]),
    "pkv_paged_decode": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i32, _i32,
                                        _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz,
                                        _i32, _vp]),
    "pkv_decode_plan": (ctypes.c_int, [_vp, _sz, _vp, _i64, _i32, _i32, _i32, _i32, _i32, _vp]),
    "pkv_paged_decode_planned": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i32,
                                                _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                                                _vp, _sz, _i32, _vp]),
    "pkv_append_paged_decode": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp,
                                               _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                               _i32, _f32, _i32, _vp, _sz, _i32, _vp]),
    "pkv_append_paged_decode_static": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64,
                                                      _vp, _vp, _i32, _vp, _i32, _i32, _i32,
                                                      _i32, _i32, _i32, _i32, _f32, _i32, _i32,
                                                      _vp]),
    "pkv_append_paged_decode_planned": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                       _i64, _vp, _vp, _i32, _vp, _i32, _i32,
                                                       _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                                                       _vp, _sz, _i32, _vp]),
    "pkv_append_paged_decode_planned_layers": (ctypes.c_int, [
        _i32, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _vp, _i64, _vp, _vp, _i64, _vp, _i64, _vp,
        _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz, _i32,
        _vp]),
    "pkv_shared_prefix_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "pkv_paged_decode_shared_prefix": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp,
                                                      _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                                      _i32, _i32, _i32, _f32, _i32, _vp, _sz,
                                                      _i32, _vp]),
    "pkv_append_paged_decode_shared_prefix": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                             _vp, _i64, _vp, _vp, _i32, _vp,
                                                             _vp, _vp, _i32, _i32, _i32, _i32,
                                                             _i32, _i32, _i32, _i32, _i32, _f32,
                                                             _i32, _vp, _sz, _i32, _vp]),
    "pkv_paged_prefill": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _i32, _i32,
                                         _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp]),
    "pkv_paged_decode_partials": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _i32,
                                                 _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                                                 _i32, _i32, _vp, _i32, _vp]),
    "pkv_lse_combine": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                       _vp]),
    "pkv_copy_blocks": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                       _i64, _i32, _vp]),
    "pkv_device_error": (ctypes.c_int, [_vp, _pi32]),
    "pkv_bm_create": (ctypes.c_int, [_i32, _i32, _vp, ctypes.POINTER(_vp)]),
    "pkv_bm_destroy": (None, [_vp]),
    "pkv_bm_add_sequence": (ctypes.c_int, [_vp, _pi32]),
    "pkv_bm_prepare_write": (ctypes.c_int, [_vp, _i32, _i32, _i32, _pi32, _pi32, _i32, _pi32]),
    "pkv_bm_prepare_step": (ctypes.c_int, [_vp, _pi32, _pi32, _pi32, _i32, _pi32, _i32, _i32,
                                           _pi32, _pi32, _i32, _pi32, _pi32]),
    "pkv_bm_fork": (ctypes.c_int, [_vp, _i32, _pi32]),
    "pkv_bm_free_sequence": (ctypes.c_int, [_vp, _i32]),
    "pkv_bm_num_blocks_of": (ctypes.c_int, [_vp, _i32, _pi32]),
    "pkv_bm_fill_tables": (ctypes.c_int, [_vp, _pi32, _i32, _pi32, _i32, _i32]),
    "pkv_bm_refcount": (ctypes.c_int, [_vp, _i32, _pi32]),
    "pkv_bm_num_free": (ctypes.c_int, [_vp, _pi32]),
    "pkv_bm_free_list": (ctypes.c_int, [_vp, _pi32, _i32, _pi32]),
    "pkv_replay_allocator": (ctypes.c_int, [_i32, _i32, _pi32, _pi32, _i32, _i32, _i32, _vp,
                                            _vp, _pi32, _i32, _vp]),
}


class ReplayResultC(ctypes.Structure):
    """pkv_replay_result (include/pkv_replay.h)."""

    _fields_ = [("peak_slots", ctypes.c_int64), ("mean_utilisation", ctypes.c_double),
                ("steps", ctypes.c_int32), ("preemptions", ctypes.c_int32)]


class PkvError(RuntimeError):
    """A libpkv call returned a negative status."""

    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed: {message} (status {status})")
        self.status = status


_LIB = None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"libpkv.so is not built ({LIB_PATH}); run "
                "`python -m paged_kv_cache_200_amd.build` (hipcc, gfx950)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def check(fn_name: str, status: int) -> None:
    if status != PKV_OK:
        msg = lib().pkv_status_string(status).decode()
        raise PkvError(fn_name, status, msg)


def call(fn_name: str, *args) -> None:
    check(fn_name, getattr(lib(), fn_name)(*args))
