"""Torch-tensor front end of libpkv: argument marshalling only.

Every function checks the tensors' device, dtype, shape and contiguity, then
passes raw device pointers and sizes to the C ABI, enqueued on the `stream`
argument (default: torch's current HIP stream).  Outputs and workspaces the
wrapper allocates itself are recorded on that stream, so the caching allocator
does not reuse them while its kernels still run.  All computation happens in
the library's kernels.

bfloat16 data may be given as torch.bfloat16 or as torch.uint16/int16 bit
patterns.
"""

from __future__ import annotations

import math

import torch

from . import _lib

BLOCK_SIZE = 16
# pkv_paged_decode merges a split sequence inside its first pass up to this many
# partitions, and in a second (combine) launch past it (include/pkv.h)
IN_PASS_MERGE_MAX_PARTITIONS = 8
_BF16_TYPES = (torch.bfloat16, torch.uint16, torch.int16)


def _kv_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return _lib.PKV_F32
    if t.dtype in _BF16_TYPES:
        return _lib.PKV_BF16
    raise TypeError(f"unsupported K/V dtype {t.dtype} (float32 or bfloat16)")


def _same_kind(a: torch.Tensor, b: torch.Tensor, what: str):
    if _kv_code(a) != _kv_code(b):
        raise TypeError(f"{what}: dtype {a.dtype} does not match {b.dtype}")


def _gpu(t: torch.Tensor, what: str, dtype=None, contiguous=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if not t.is_cuda:  # an attribute read: a third of the cost of t.device.type
        raise ValueError(f"{what} must be on the GPU (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype} (got {t.dtype})")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _held(t, stream):
    """A tensor the wrapper allocated, used by kernels on `stream`: when that is not torch's
    current stream, tell the caching allocator, so the memory is not handed out again
    before the stream's work on it is done."""
    if t is not None and stream is not None and stream != torch.cuda.current_stream(t.device):
        t.record_stream(stream)
    return t


def _ptr(t):
    return None if t is None else t.data_ptr()


def _cache_dims(k_cache: torch.Tensor):
    if k_cache.dim() != 4 or k_cache.shape[2] != BLOCK_SIZE:
        raise ValueError("caches must be [num_blocks, num_kv_heads, 16, head_dim]")
    nb, hkv, _, d = k_cache.shape
    return nb, hkv, d


def kv_append(k_cache, v_cache, k_new, v_new, block_tables, start_pos, cu_new_tokens,
              stream=None) -> None:
    """Write k_new/v_new [T, Hkv, D] at positions start_pos[s] + i (explicit, never inferred)."""
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache"), (k_new, "k_new"), (v_new, "v_new")):
        _gpu(t, n)
    _same_kind(k_cache, v_cache, "v_cache")
    _same_kind(k_cache, k_new, "k_new")
    _same_kind(k_cache, v_new, "v_new")
    nb, hkv, d = _cache_dims(k_cache)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    if k_new.dim() != 3 or tuple(k_new.shape[1:]) != (hkv, d) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [T, num_kv_heads, head_dim]")
    _gpu(block_tables, "block_tables", torch.int32)
    _gpu(start_pos, "start_pos", torch.int32)
    _gpu(cu_new_tokens, "cu_new_tokens", torch.int32)
    B = start_pos.shape[0]
    if block_tables.dim() != 2 or block_tables.shape[0] != B or cu_new_tokens.shape[0] != B + 1:
        raise ValueError("block_tables [B, W], start_pos [B], cu_new_tokens [B + 1] expected")
    _lib.call("pkv_kv_append", _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
              _ptr(block_tables), block_tables.shape[1], _ptr(start_pos), _ptr(cu_new_tokens),
              B, k_new.shape[0], hkv, d, BLOCK_SIZE, nb, _kv_code(k_cache), _stream(stream))


def decode_workspace_bytes(batch, num_q_heads, head_dim, max_context_len, partition_size) -> int:
    return int(_lib.lib().pkv_decode_workspace_bytes(batch, num_q_heads, head_dim,
                                                     max_context_len, partition_size))


def decode_partition_size(batch, num_kv_heads, head_dim, max_context_len,
                          total_context_tokens=0) -> int:
    """The library's partition-size rule (pkv_decode_partition_size): 0 (no split) or a
    power of two from the call's size; total_context_tokens <= 0 assumes every sequence
    is max_context_len long."""
    return int(_lib.lib().pkv_decode_partition_size(batch, num_kv_heads, head_dim,
                                                    int(max_context_len),
                                                    int(total_context_tokens)))


def decode_engine(kv_dtype, head_dim, num_q_heads, num_kv_heads) -> str:
    """Which first pass the decode calls run for these shapes (pkv_decode_engine):
    "valu" (decode_pass1_kernel) or "matrix" (the bf16 matrix-core tile)."""
    codes = {"f32": _lib.PKV_F32, "bf16": _lib.PKV_BF16}
    if kv_dtype not in codes:
        raise TypeError(f"unsupported K/V dtype {kv_dtype!r} ('f32' or 'bf16')")
    code = int(_lib.lib().pkv_decode_engine(codes[kv_dtype], head_dim, num_q_heads,
                                            num_kv_heads))
    if code < 0:
        _lib.check("pkv_decode_engine", code)
    return "matrix" if code == 1 else "valu"


def shared_prefix_workspace_bytes(batch, num_q_heads, head_dim, max_context_len,
                                  partition_size) -> int:
    return int(_lib.lib().pkv_shared_prefix_workspace_bytes(batch, num_q_heads, head_dim,
                                                            max_context_len, partition_size))


def _decode_checks(q, k_cache, v_cache, block_tables, context_lens):
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _gpu(t, n)
    _same_kind(k_cache, v_cache, "v_cache")
    _same_kind(k_cache, q, "q")
    nb, hkv, d = _cache_dims(k_cache)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    if q.dim() != 3 or q.shape[2] != d:
        raise ValueError("q must be [batch, num_q_heads, head_dim]")
    B, hq, _ = q.shape
    _gpu(block_tables, "block_tables", torch.int32)
    _gpu(context_lens, "context_lens", torch.int32)
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables [B, W] and context_lens [B] expected")
    return B, hq, hkv, d, nb


def _workspace(workspace, need, device, stream=None):
    if workspace is None:
        workspace = _held(torch.empty(max(need, 1), dtype=torch.uint8, device=device), stream)
    _gpu(workspace, "workspace")
    wbytes = workspace.numel() * workspace.element_size()
    if wbytes < need:
        raise ValueError(f"workspace holds {wbytes} bytes, {need} needed")
    if workspace.data_ptr() % 256:
        raise ValueError("workspace must be 256-byte aligned")
    return workspace, wbytes


def decode_plan(context_lens, block_tables, num_q_heads, head_dim, max_context_len,
                partition_size=0, workspace=None, stream=None):
    """Write the first pass's longest-first work plan into a (new or given) workspace."""
    _gpu(context_lens, "context_lens", torch.int32)
    _gpu(block_tables, "block_tables", torch.int32)
    B = context_lens.shape[0]
    need = decode_workspace_bytes(B, num_q_heads, head_dim, max_context_len, partition_size)
    workspace, wbytes = _workspace(workspace, need, context_lens.device, stream)
    _lib.call("pkv_decode_plan", _ptr(workspace), wbytes, _ptr(context_lens),
              block_tables.shape[1], B, num_q_heads, head_dim, int(max_context_len),
              int(partition_size), _stream(stream))
    return workspace


def _decode(fn_name, q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
            partition_size, out, lse, workspace, want_lse, stream):
    B, hq, hkv, d, nb = _decode_checks(q, k_cache, v_cache, block_tables, context_lens)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _outputs(out, lse, want_lse, B, hq, d, q.device, stream)
    need = decode_workspace_bytes(B, hq, d, max_context_len, partition_size)
    workspace, wbytes = _workspace(workspace, need, q.device, stream)
    _lib.call(fn_name, _ptr(out), _ptr(lse), _ptr(q), _ptr(k_cache), _ptr(v_cache),
              _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), B, hq, hkv, d,
              BLOCK_SIZE, nb, int(max_context_len), float(scale), int(partition_size),
              _ptr(workspace), wbytes, _kv_code(k_cache), _stream(stream))
    return out, lse


def paged_decode(q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale=None,
                 partition_size=0, out=None, lse=None, workspace=None, want_lse=True,
                 stream=None):
    """Decode attention of q [B, Hq, D] over the paged caches (plan, then a first pass that
    also merges the partitions of split sequences).

    Returns (out float32 [B, Hq, D], lse float32 [B, Hq] or None).
    max_context_len is a host-side upper bound of context_lens.
    """
    return _decode("pkv_paged_decode", q, k_cache, v_cache, block_tables, context_lens,
                   max_context_len, scale, partition_size, out, lse, workspace, want_lse, stream)


def paged_decode_planned(q, k_cache, v_cache, block_tables, context_lens, max_context_len,
                         workspace, scale=None, partition_size=0, out=None, lse=None,
                         want_lse=True, stream=None):
    """paged_decode reusing a plan already written into `workspace` by decode_plan."""
    if workspace is None:
        raise ValueError("paged_decode_planned needs the workspace decode_plan filled")
    return _decode("pkv_paged_decode_planned", q, k_cache, v_cache, block_tables, context_lens,
                   max_context_len, scale, partition_size, out, lse, workspace, want_lse, stream)


def _append_checks(k_cache, k_new, v_new, start_pos, cu_new_tokens, B, hkv, d):
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _gpu(t, n)
        _same_kind(k_cache, t, n)
    if k_new.dim() != 3 or tuple(k_new.shape[1:]) != (hkv, d) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [T, num_kv_heads, head_dim]")
    _gpu(start_pos, "start_pos", torch.int32)
    _gpu(cu_new_tokens, "cu_new_tokens", torch.int32)
    if start_pos.shape != (B,) or cu_new_tokens.shape != (B + 1,):
        raise ValueError("start_pos [B] and cu_new_tokens [B + 1] expected")


def _group_checks(group_starts, group_shared_blocks):
    _gpu(group_starts, "group_starts", torch.int32)
    _gpu(group_shared_blocks, "group_shared_blocks", torch.int32)
    G = group_shared_blocks.shape[0]
    if group_starts.shape != (G + 1,):
        raise ValueError("group_starts must have num_groups + 1 entries")
    return G


def _outputs(out, lse, want_lse, B, hq, d, device, stream=None):
    if out is None:
        out = _held(torch.empty((B, hq, d), dtype=torch.float32, device=device), stream)
    _gpu(out, "out", torch.float32)
    if lse is None and want_lse:
        lse = _held(torch.empty((B, hq), dtype=torch.float32, device=device), stream)
    if lse is not None:
        _gpu(lse, "lse", torch.float32)
    return out, lse


def append_paged_decode(q, k_cache, v_cache, k_new, v_new, block_tables, start_pos,
                        cu_new_tokens, context_lens, max_context_len, scale=None,
                        partition_size=0, out=None, lse=None, workspace=None, want_lse=True,
                        stream=None):
    """kv_append then paged_decode in one call (append and work plan share a launch).

    context_lens must already count the appended tokens.
    """
    B, hq, hkv, d, nb = _decode_checks(q, k_cache, v_cache, block_tables, context_lens)
    _append_checks(k_cache, k_new, v_new, start_pos, cu_new_tokens, B, hkv, d)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _outputs(out, lse, want_lse, B, hq, d, q.device, stream)
    need = decode_workspace_bytes(B, hq, d, max_context_len, partition_size)
    workspace, wbytes = _workspace(workspace, need, q.device, stream)
    _lib.call("pkv_append_paged_decode", _ptr(out), _ptr(lse), _ptr(q), _ptr(k_cache),
              _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(block_tables),
              block_tables.shape[1], _ptr(start_pos), _ptr(cu_new_tokens), k_new.shape[0],
              _ptr(context_lens), B, hq, hkv, d, BLOCK_SIZE, nb, int(max_context_len),
              float(scale), int(partition_size), _ptr(workspace), wbytes, _kv_code(k_cache),
              _stream(stream))
    return out, lse


def append_paged_decode_static(q, k_cache, v_cache, k_new, v_new, block_tables, start_pos,
                               cu_new_tokens, context_lens, max_context_len, out, lse=None,
                               scale=None, partition_size=0, stream=None):
    """append_paged_decode with no workspace and no allocation: the library's static
    per-GPU scratch array (STATIC_SCRATCH_BYTES) holds the plan and partial results, and
    out (and lse, optional) must be given.  Calls that overlap in time on one GPU race."""
    B, hq, hkv, d, nb = _decode_checks(q, k_cache, v_cache, block_tables, context_lens)
    _append_checks(k_cache, k_new, v_new, start_pos, cu_new_tokens, B, hkv, d)
    if out is None:
        raise ValueError("append_paged_decode_static allocates nothing: pass out")
    _gpu(out, "out", torch.float32)
    if lse is not None:
        _gpu(lse, "lse", torch.float32)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _lib.call("pkv_append_paged_decode_static", _ptr(out), _ptr(lse), _ptr(q), _ptr(k_cache),
              _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(block_tables),
              block_tables.shape[1], _ptr(start_pos), _ptr(cu_new_tokens), k_new.shape[0],
              _ptr(context_lens), B, hq, hkv, d, BLOCK_SIZE, nb, int(max_context_len),
              float(scale), int(partition_size), _kv_code(k_cache), _stream(stream))
    return out, lse


STATIC_SCRATCH_BYTES = _lib.STATIC_SCRATCH_BYTES


def append_paged_decode_planned(q, k_cache, v_cache, k_new, v_new, block_tables, start_pos,
                                cu_new_tokens, context_lens, max_context_len, workspace,
                                scale=None, partition_size=0, out=None, lse=None,
                                want_lse=True, stream=None):
    """kv_append then paged_decode in one launch, on a plan that decode_plan wrote into
    `workspace` for the same context_lens (one plan serves every layer of a step).

    context_lens must already count the appended tokens.
    """
    if workspace is None:
        raise ValueError("append_paged_decode_planned needs the workspace decode_plan filled")
    B, hq, hkv, d, nb = _decode_checks(q, k_cache, v_cache, block_tables, context_lens)
    _append_checks(k_cache, k_new, v_new, start_pos, cu_new_tokens, B, hkv, d)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _outputs(out, lse, want_lse, B, hq, d, q.device, stream)
    need = decode_workspace_bytes(B, hq, d, max_context_len, partition_size)
    workspace, wbytes = _workspace(workspace, need, q.device, stream)
    _lib.call("pkv_append_paged_decode_planned", _ptr(out), _ptr(lse), _ptr(q), _ptr(k_cache),
              _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(block_tables),
              block_tables.shape[1], _ptr(start_pos), _ptr(cu_new_tokens), k_new.shape[0],
              _ptr(context_lens), B, hq, hkv, d, BLOCK_SIZE, nb, int(max_context_len),
              float(scale), int(partition_size), _ptr(workspace), wbytes, _kv_code(k_cache),
              _stream(stream))
    return out, lse


class DecodeStep:
    """One decode step over the layers of a model: append_paged_decode_planned per layer,
    with the host work of a call cut to what differs between layers.

    The constructor takes the first layer's tensors and checks everything as
    append_paged_decode_planned does.  The step-wide tensors (block tables, positions,
    cu_new_tokens, context lengths, plan workspace, default outputs) are bound here, and
    the work plan is written for them (plan=True).  layer() then checks only what a layer
    brings: its q, caches and new K/V must have the first layer's shapes, dtype kind and
    device, and be contiguous.  Each layer() is one pkv_append_paged_decode_planned call
    (a single launch while no sequence has more than IN_PASS_MERGE_MAX_PARTITIONS
    partitions), with the same results as the function.

    partition_size None (the default) takes the library's rule (decode_partition_size),
    from max_context_len and, when given, the step's total_context_tokens.

    Bound tensors must stay allocated and keep their shapes while the object is used.
    Their contents may change in place between steps; plan() must then run again before
    the next layer().  Results go to the bound out/lse unless a layer passes its own.
    """

    def __init__(self, q, k_cache, v_cache, k_new, v_new, block_tables, start_pos,
                 cu_new_tokens, context_lens, max_context_len, scale=None, partition_size=None,
                 out=None, lse=None, want_lse=True, workspace=None, stream=None, plan=True,
                 total_context_tokens=0):
        B, hq, hkv, d, nb = _decode_checks(q, k_cache, v_cache, block_tables, context_lens)
        if partition_size is None:
            partition_size = decode_partition_size(B, hkv, d, max_context_len,
                                                   total_context_tokens)
        _append_checks(k_cache, k_new, v_new, start_pos, cu_new_tokens, B, hkv, d)
        if scale is None:
            scale = 1.0 / math.sqrt(d)
        self.out, self.lse = _outputs(out, lse, want_lse, B, hq, d, q.device, stream)
        need = decode_workspace_bytes(B, hq, d, max_context_len, partition_size)
        self.workspace, wbytes = _workspace(workspace, need, q.device, stream)
        self.block_tables, self.start_pos = block_tables, start_pos
        self.cu_new_tokens, self.context_lens = cu_new_tokens, context_lens
        self.max_context_len = int(max_context_len)
        self.partition_size = int(partition_size)
        self.num_q_heads, self.head_dim = hq, d
        self.stream = stream
        self._q_shape, self._cache_shape, self._new_shape = q.shape, k_cache.shape, k_new.shape
        self._out_shape, self._lse_shape = (B, hq, d), (B, hq)
        self._kinds = (torch.float32,) if k_cache.dtype == torch.float32 else _BF16_TYPES
        self._device = q.get_device()
        self._fn = getattr(_lib.lib(), "pkv_append_paged_decode_planned")
        self._fixed = (block_tables.data_ptr(), block_tables.shape[1], start_pos.data_ptr(),
                       cu_new_tokens.data_ptr(), k_new.shape[0], context_lens.data_ptr(), B,
                       hq, hkv, d, BLOCK_SIZE, nb, self.max_context_len, float(scale),
                       self.partition_size, self.workspace.data_ptr(), wbytes,
                       _kv_code(k_cache))
        if plan:
            self.plan()

    def plan(self):
        """(Re)write the work plan for the bound context lengths and tables."""
        decode_plan(self.context_lens, self.block_tables, self.num_q_heads, self.head_dim,
                    self.max_context_len, self.partition_size, workspace=self.workspace,
                    stream=self.stream)

    def _check(self, t, shape, kinds, what):
        if (not isinstance(t, torch.Tensor) or t.shape != shape or t.dtype not in kinds
                or t.get_device() != self._device or not t.is_contiguous()):
            kind = "float32" if kinds[0] == torch.float32 else "bfloat16 (or its bits)"
            raise ValueError(f"{what} must be a contiguous {kind} tensor of shape "
                             f"{tuple(shape)} on GPU {self._device}, like the first layer's")

    def layer(self, q, k_cache, v_cache, k_new, v_new, out=None, lse=None):
        """Append this layer's new tokens to its caches and attend; returns (out, lse)."""
        kinds = self._kinds
        self._check(q, self._q_shape, kinds, "q")
        self._check(k_cache, self._cache_shape, kinds, "k_cache")
        self._check(v_cache, self._cache_shape, kinds, "v_cache")
        self._check(k_new, self._new_shape, kinds, "k_new")
        self._check(v_new, self._new_shape, kinds, "v_new")
        if out is None:
            out = self.out
        else:
            self._check(out, self._out_shape, (torch.float32,), "out")
        if lse is None:
            lse = self.lse
        else:
            self._check(lse, self._lse_shape, (torch.float32,), "lse")
        s = torch.cuda.current_stream() if self.stream is None else self.stream
        _lib.check("pkv_append_paged_decode_planned",
                   self._fn(out.data_ptr(), None if lse is None else lse.data_ptr(),
                            q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                            k_new.data_ptr(), v_new.data_ptr(), *self._fixed, s.cuda_stream))
        return out, lse

    def layers(self, q, k_cache, v_cache, k_new, v_new, out=None, lse=None):
        """Every layer of the step in one library call
        (pkv_append_paged_decode_planned_layers): the tensors stack the layers on a
        leading dimension (q [L, *q], caches [L, *cache], new K/V [L, *new], each layer
        shaped like the first layer's); outputs go to out / lse stacked the same way, or
        to the bound out / lse, which every layer then overwrites.  Same results as
        layer() on each slice in order; returns (out, lse)."""
        kinds = self._kinds
        L = q.shape[0] if isinstance(q, torch.Tensor) and q.dim() > 0 else -1
        self._check(q, (L,) + tuple(self._q_shape), kinds, "q")
        self._check(k_cache, (L,) + tuple(self._cache_shape), kinds, "k_cache")
        self._check(v_cache, (L,) + tuple(self._cache_shape), kinds, "v_cache")
        self._check(k_new, (L,) + tuple(self._new_shape), kinds, "k_new")
        self._check(v_new, (L,) + tuple(self._new_shape), kinds, "v_new")
        out_stride, lse_stride = 0, 0
        if out is None:
            out = self.out
        else:
            self._check(out, (L,) + tuple(self._out_shape), (torch.float32,), "out")
            out_stride = out.stride(0)
        if lse is None:
            lse = self.lse
        else:
            self._check(lse, (L,) + tuple(self._lse_shape), (torch.float32,), "lse")
            lse_stride = lse.stride(0)
        s = torch.cuda.current_stream() if self.stream is None else self.stream
        _lib.call("pkv_append_paged_decode_planned_layers", L, out.data_ptr(), out_stride,
                  None if lse is None else lse.data_ptr(), lse_stride, q.data_ptr(),
                  q.stride(0), k_cache.data_ptr(), v_cache.data_ptr(), k_cache.stride(0),
                  k_new.data_ptr(), v_new.data_ptr(), k_new.stride(0), *self._fixed,
                  s.cuda_stream)
        return out, lse


def append_paged_decode_layers(q, k_cache, v_cache, k_new, v_new, block_tables, start_pos,
                               cu_new_tokens, context_lens, max_context_len, workspace,
                               scale=None, partition_size=0, out=None, lse=None, stream=None):
    """A whole decode step over stacked layers in two library calls: pkv_decode_plan for the
    step's lengths, then pkv_append_paged_decode_planned_layers (each layer's append +
    decode in order).  q [L, B, Hq, D], caches [L, NB, Hkv, 16, D], k_new / v_new
    [L, T, Hkv, D]; out [B, Hq, D] (every layer overwrites it, the last layer's result
    stays) or [L, B, Hq, D]; lse likewise, or None.  Same results as DecodeStep.layers.
    The tensors are checked once for the step, the workspace size by the library."""
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (k_new, "k_new"),
                 (v_new, "v_new")):
        _gpu(t, n)
        _same_kind(k_cache, t, n)
    if q.dim() != 4 or k_cache.dim() != 5 or k_new.dim() != 4:
        raise ValueError("stacked tensors expected: q [L, B, Hq, D], caches "
                         "[L, NB, Hkv, 16, D], k_new / v_new [L, T, Hkv, D]")
    L, B, hq, d = q.shape
    _, nb, hkv, bs, dk = k_cache.shape
    if (v_cache.shape != k_cache.shape or k_cache.shape[0] != L or bs != BLOCK_SIZE
            or dk != d or v_new.shape != k_new.shape or k_new.shape[0] != L
            or tuple(k_new.shape[2:]) != (hkv, d)):
        raise ValueError("q, caches and new K/V must stack the same layers and heads")
    for t, n in ((block_tables, "block_tables"), (start_pos, "start_pos"),
                 (cu_new_tokens, "cu_new_tokens"), (context_lens, "context_lens")):
        _gpu(t, n, torch.int32)
    if (block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,)
            or start_pos.shape != (B,) or cu_new_tokens.shape != (B + 1,)):
        raise ValueError("block_tables [B, W], start_pos / context_lens [B] and "
                         "cu_new_tokens [B + 1] expected")
    _gpu(workspace, "workspace")
    if out is None:
        raise ValueError("out is required: [B, Hq, D] or [L, B, Hq, D] float32")
    _gpu(out, "out", torch.float32)
    if tuple(out.shape) == (B, hq, d):
        out_stride = 0
    elif tuple(out.shape) == (L, B, hq, d):
        out_stride = out.stride(0)
    else:
        raise ValueError("out must be [B, Hq, D] or [L, B, Hq, D]")
    lse_stride = 0
    if lse is not None:
        _gpu(lse, "lse", torch.float32)
        if tuple(lse.shape) == (L, B, hq):
            lse_stride = lse.stride(0)
        elif tuple(lse.shape) != (B, hq):
            raise ValueError("lse must be [B, Hq] or [L, B, Hq]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    wbytes = workspace.numel() * workspace.element_size()
    st = _stream(stream)
    W = block_tables.shape[1]
    _lib.call("pkv_decode_plan", workspace.data_ptr(), wbytes, context_lens.data_ptr(), W, B,
              hq, d, int(max_context_len), int(partition_size), st)
    _lib.call("pkv_append_paged_decode_planned_layers", L, out.data_ptr(), out_stride,
              _ptr(lse), lse_stride, q.data_ptr(), q.stride(0), k_cache.data_ptr(),
              v_cache.data_ptr(), k_cache.stride(0), k_new.data_ptr(), v_new.data_ptr(),
              k_new.stride(0), block_tables.data_ptr(), W, start_pos.data_ptr(),
              cu_new_tokens.data_ptr(), k_new.shape[1], context_lens.data_ptr(), B, hq, hkv,
              d, BLOCK_SIZE, nb, int(max_context_len), float(scale), int(partition_size),
              workspace.data_ptr(), wbytes, _kv_code(k_cache), st)
    return out, lse


def paged_decode_shared_prefix(q, k_cache, v_cache, block_tables, context_lens, group_starts,
                               group_shared_blocks, max_shared_blocks, max_context_len,
                               scale=None, partition_size=0, out=None, lse=None, workspace=None,
                               want_lse=True, stream=None):
    """Decode a batch of copy-on-write fork groups, streaming each group's shared
    leading blocks once for all members (see pkv_paged_decode_shared_prefix)."""
    B, hq, hkv, d, nb = _decode_checks(q, k_cache, v_cache, block_tables, context_lens)
    G = _group_checks(group_starts, group_shared_blocks)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _outputs(out, lse, want_lse, B, hq, d, q.device, stream)
    need = shared_prefix_workspace_bytes(B, hq, d, int(max_context_len), int(partition_size))
    workspace, wbytes = _workspace(workspace, need, q.device, stream)
    _lib.call("pkv_paged_decode_shared_prefix", _ptr(out), _ptr(lse), _ptr(q), _ptr(k_cache),
              _ptr(v_cache), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
              _ptr(group_starts), _ptr(group_shared_blocks), G, int(max_shared_blocks), B, hq,
              hkv, d, BLOCK_SIZE, nb, int(max_context_len), float(scale), int(partition_size),
              _ptr(workspace), wbytes, _kv_code(k_cache), _stream(stream))
    return out, lse


def append_paged_decode_shared_prefix(q, k_cache, v_cache, k_new, v_new, block_tables,
                                      start_pos, cu_new_tokens, context_lens, group_starts,
                                      group_shared_blocks, max_shared_blocks, max_context_len,
                                      scale=None, partition_size=0, out=None, lse=None,
                                      workspace=None, want_lse=True, stream=None):
    """kv_append then paged_decode_shared_prefix, append and work plan in one launch.
    New tokens must not land in a block that several sequences hold."""
    B, hq, hkv, d, nb = _decode_checks(q, k_cache, v_cache, block_tables, context_lens)
    _append_checks(k_cache, k_new, v_new, start_pos, cu_new_tokens, B, hkv, d)
    G = _group_checks(group_starts, group_shared_blocks)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out, lse = _outputs(out, lse, want_lse, B, hq, d, q.device, stream)
    need = shared_prefix_workspace_bytes(B, hq, d, int(max_context_len), int(partition_size))
    workspace, wbytes = _workspace(workspace, need, q.device, stream)
    _lib.call("pkv_append_paged_decode_shared_prefix", _ptr(out), _ptr(lse), _ptr(q),
              _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(block_tables),
              block_tables.shape[1], _ptr(start_pos), _ptr(cu_new_tokens), k_new.shape[0],
              _ptr(context_lens), _ptr(group_starts), _ptr(group_shared_blocks), G,
              int(max_shared_blocks), B, hq, hkv, d, BLOCK_SIZE, nb, int(max_context_len),
              float(scale), int(partition_size), _ptr(workspace), wbytes, _kv_code(k_cache),
              _stream(stream))
    return out, lse


def paged_prefill(q, k_cache, v_cache, block_tables, cu_q, context_lens, max_q_len,
                  scale=None, out=None, lse=None, want_lse=True, stream=None):
    """Causal attention of each sequence's newest chunk of query tokens over its paged
    context (see pkv_paged_prefill).  q [T, Hq, D]; returns (out [T, Hq, D], lse [T, Hq])
    float32.  The chunk's K/V must already be appended."""
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _gpu(t, n)
    _same_kind(k_cache, q, "q")
    _same_kind(k_cache, v_cache, "v_cache")
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q [T, Hq, D] and caches [NB, Hkv, 16, D] expected")
    T, hq, d = q.shape
    nb, hkv = k_cache.shape[0], k_cache.shape[1]
    if k_cache.shape[2] != BLOCK_SIZE or k_cache.shape[3] != d:
        raise ValueError("cache must be [num_blocks, num_kv_heads, 16, head_dim]")
    _gpu(block_tables, "block_tables", torch.int32)
    _gpu(cu_q, "cu_q", torch.int32)
    _gpu(context_lens, "context_lens", torch.int32)
    B = context_lens.shape[0]
    if cu_q.shape != (B + 1,) or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("cu_q [B + 1] and block_tables [B, W] expected")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = _held(torch.empty((T, hq, d), dtype=torch.float32, device=q.device), stream)
    _gpu(out, "out", torch.float32)
    if lse is None and want_lse:
        lse = _held(torch.empty((T, hq), dtype=torch.float32, device=q.device), stream)
    if lse is not None:
        _gpu(lse, "lse", torch.float32)
    _lib.call("pkv_paged_prefill", _ptr(out), _ptr(lse), _ptr(q), _ptr(k_cache), _ptr(v_cache),
              _ptr(block_tables), block_tables.shape[1], _ptr(cu_q), _ptr(context_lens), B, T,
              int(max_q_len), hq, hkv, d, BLOCK_SIZE, nb, float(scale), _kv_code(k_cache),
              _stream(stream))
    return out, lse


def paged_decode_partials(q, k_cache, v_cache, block_tables, context_lens, max_context_len,
                          partition_size, scale=None, max_partitions=None, part_out=None,
                          part_lse=None, plan_workspace=None, stream=None):
    """First pass only: (part_out [B, Hq, NP, D], part_lse [B, Hq, NP]) float32.

    plan_workspace: optional workspace holding a decode_plan for the same inputs and
    partition_size; the pass then runs in the plan's order.
    """
    B, hq, hkv, d, nb = _decode_checks(q, k_cache, v_cache, block_tables, context_lens)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if partition_size <= 0:
        raise ValueError("partition_size must be positive")
    np_ = max(1, -(-int(max_context_len) // int(partition_size)))
    if max_partitions is None:
        max_partitions = np_
    if part_out is None:
        part_out = _held(torch.empty((B, hq, max_partitions, d), dtype=torch.float32,
                                     device=q.device), stream)
    if part_lse is None:
        part_lse = _held(torch.empty((B, hq, max_partitions), dtype=torch.float32,
                                     device=q.device), stream)
    _gpu(part_out, "part_out", torch.float32)
    _gpu(part_lse, "part_lse", torch.float32)
    _lib.call("pkv_paged_decode_partials", _ptr(part_out), _ptr(part_lse), _ptr(q),
              _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), block_tables.shape[1],
              _ptr(context_lens), B, hq, hkv, d, BLOCK_SIZE, nb, int(max_context_len),
              float(scale), int(partition_size), int(max_partitions), _ptr(plan_workspace),
              _kv_code(k_cache), _stream(stream))
    return part_out, part_lse


def lse_combine(part_out, part_lse, context_lens, partition_size, out=None, lse=None,
                want_lse=True, stream=None):
    """Merge partitions by log-sum-exp: (out [B, Hq, D], lse [B, Hq])."""
    _gpu(part_out, "part_out", torch.float32)
    _gpu(part_lse, "part_lse", torch.float32)
    _gpu(context_lens, "context_lens", torch.int32)
    if part_out.dim() != 4 or part_lse.shape != part_out.shape[:3]:
        raise ValueError("part_out [B, Hq, NP, D] and part_lse [B, Hq, NP] expected")
    B, hq, np_, d = part_out.shape
    if out is None:
        out = _held(torch.empty((B, hq, d), dtype=torch.float32, device=part_out.device), stream)
    if lse is None and want_lse:
        lse = _held(torch.empty((B, hq), dtype=torch.float32, device=part_out.device), stream)
    _gpu(out, "out", torch.float32)
    _lib.call("pkv_lse_combine", _ptr(out), _ptr(lse), _ptr(part_out), _ptr(part_lse),
              _ptr(context_lens), B, hq, d, int(partition_size), np_, _stream(stream))
    return out, lse


def copy_blocks(k_cache, v_cache, src, dst, stream=None) -> None:
    """Copy-on-write block copy: block dst[i] := block src[i] in both caches.

    Caches may be one layer [NB, Hkv, 16, D] or stacked layers [L, NB, Hkv, 16, D]
    (every layer copied).
    """
    _gpu(k_cache, "k_cache")
    _gpu(v_cache, "v_cache")
    _same_kind(k_cache, v_cache, "v_cache")
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    if k_cache.dim() == 5:
        layers = k_cache.shape[0]
        layer_stride = k_cache.stride(0)
        nb, hkv, d = _cache_dims(k_cache[0])
    else:
        layers, layer_stride = 1, 0
        nb, hkv, d = _cache_dims(k_cache)
    _gpu(src, "src", torch.int32)
    _gpu(dst, "dst", torch.int32)
    if src.shape != dst.shape or src.dim() != 1:
        raise ValueError("src and dst must be equal-length int32 vectors")
    _lib.call("pkv_copy_blocks", _ptr(k_cache), _ptr(v_cache), _ptr(src), _ptr(dst),
              src.shape[0], hkv, d, BLOCK_SIZE, nb, layers, layer_stride, _kv_code(k_cache),
              _stream(stream))


def device_error(stream=None) -> int:
    """Synchronise the stream and return (and clear) the device error bits."""
    flags = _lib._i32(0)
    _lib.call("pkv_device_error", _stream(stream), _lib.ctypes.byref(flags))
    return int(flags.value)


def describe_device_error(flags: int) -> str:
    return ", ".join(v for k, v in _lib.DEVICE_ERROR_BITS.items() if flags & k) or "none"
