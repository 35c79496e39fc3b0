"""Python binding over the C ABI (argument marshalling only).

Tensors are used as device memory; every call is enqueued on torch's current
HIP stream.  All arithmetic runs in the library's kernels.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib

_DTYPE = {torch.float32: _lib.PA_F32, torch.float16: _lib.PA_F16,
          torch.bfloat16: _lib.PA_BF16}


def _dt(t: torch.Tensor) -> int:
    try:
        return _DTYPE[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("paged decode attention runs on the GPU: pass device tensors")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping) -> None:
    """Write key[i]/value[i] ([T, Hkv, D]) into slot slot_mapping[i] (int64,
    -1 = skip) of the paged caches ([NB, bs, Hkv, D]), in place."""
    _dev(key, value, k_cache, v_cache, slot_mapping)
    if slot_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping must be int64")
    if not (key.dtype == value.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("key, value and caches must share a dtype")
    NB, bs, Hkv, D = k_cache.shape
    if tuple(v_cache.shape) != (NB, bs, Hkv, D):
        raise ValueError("k_cache and v_cache shapes differ")
    T = key.shape[0]
    if tuple(key.shape) != (T, Hkv, D) or tuple(value.shape) != (T, Hkv, D) \
            or tuple(slot_mapping.shape) != (T,):
        raise ValueError("key/value must be [T, Hkv, D] and slot_mapping [T]")
    lib = _lib.load()
    _lib.check("pa_reshape_and_cache", lib.pa_reshape_and_cache(
        key.data_ptr(), value.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        slot_mapping.data_ptr(), T, NB, bs, Hkv, D, _dt(key), _stream()))


def copy_blocks(k_cache, v_cache, block_mapping) -> None:
    """Copy whole blocks src -> dst in both caches, in place; block_mapping is
    int64 [num_pairs, 2] of (src, dst) physical block ids."""
    _dev(k_cache, v_cache, block_mapping)
    if block_mapping.dtype != torch.int64 or block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be int64 [num_pairs, 2]")
    if k_cache.dtype != v_cache.dtype or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must match")
    NB, bs, Hkv, D = k_cache.shape
    _lib.check("pa_copy_blocks", _lib.load().pa_copy_blocks(
        k_cache.data_ptr(), v_cache.data_ptr(), block_mapping.data_ptr(),
        block_mapping.shape[0], NB, bs, Hkv, D, _dt(k_cache), _stream()))


def partition_size(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                   max_context_len, window=0, dtype=torch.bfloat16) -> int:
    """The library's choice of split-K partition size for a shape."""
    return int(_lib.load().pa_decode_partition_size(
        num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_context_len,
        window, _DTYPE[dtype]))


def workspace_size(num_seqs, num_heads, head_dim, max_context_len, partition_size) -> int:
    return int(_lib.load().pa_decode_workspace_size(
        num_seqs, num_heads, head_dim, max_context_len, partition_size))


def _shapes(q, k_cache, block_tables):
    B, Hq, D = q.shape
    NB, bs, Hkv, D2 = k_cache.shape
    if D2 != D:
        raise ValueError("head_dim of q and caches differ")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [num_seqs, max_blocks_per_seq]")
    return B, Hq, D, NB, bs, Hkv


def decode_partitions(out, workspace, q, k_cache, v_cache, block_tables, context_lens,
                      max_context_len, scale, softcap, window, partition_size) -> None:
    """pa_decode: the partition pass (writes `out` for single-partition
    sequences and split-K partials to `workspace` for the others)."""
    _dev(out, workspace, q, k_cache, v_cache, block_tables, context_lens)
    B, Hq, D, NB, bs, Hkv = _shapes(q, k_cache, block_tables)
    if context_lens.dtype != torch.int32 or tuple(context_lens.shape) != (B,):
        raise ValueError("context_lens must be int32 [num_seqs]")
    if not (q.dtype == k_cache.dtype == v_cache.dtype == out.dtype):
        raise TypeError("q, caches and out must share a dtype")
    if tuple(out.shape) != (B, Hq, D):
        raise ValueError("out must be [num_seqs, num_heads, head_dim]")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    lib = _lib.load()
    _lib.check("pa_decode", lib.pa_decode(
        out.data_ptr(), ws_ptr, ws_bytes, q.data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), block_tables.data_ptr(), block_tables.shape[1],
        context_lens.data_ptr(), int(max_context_len), B, Hq, Hkv, D, bs, NB,
        float(scale), float(softcap), int(window), int(partition_size), _dt(q), _stream()))


def set_decode_events(start=None, stop=None) -> None:
    """Have this thread's pa_decode calls record ``start`` / ``stop``
    (torch.cuda.Event objects, each recorded once before so that it exists)
    right around their decode kernel; no arguments clears."""
    if (start is None) != (stop is None):
        raise ValueError("give both events or neither")
    _lib.check("pa_set_decode_events", _lib.load().pa_set_decode_events(
        start.cuda_event if start is not None else None,
        stop.cuda_event if stop is not None else None))


def read_bandwidth_probe(buf, grid, sink) -> None:
    """pa_read_bandwidth_probe: one streaming read of the device tensor
    ``buf`` (its whole storage, a multiple of 16 bytes) by ``grid``
    workgroups, queued on torch's current stream; ``sink`` is a device
    tensor of at least 4 bytes the kernel may write."""
    _dev(buf, sink)
    nbytes = buf.numel() * buf.element_size()
    _lib.check("pa_read_bandwidth_probe", _lib.load().pa_read_bandwidth_probe(
        buf.data_ptr(), nbytes, int(grid), sink.data_ptr(), _stream()))


def decode_reduce(out, workspace, context_lens, max_context_len, partition_size,
                  window) -> None:
    """pa_decode_reduce: merge the partials of multi-partition sequences."""
    _dev(out, workspace, context_lens)
    B, Hq, D = out.shape
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    lib = _lib.load()
    _lib.check("pa_decode_reduce", lib.pa_decode_reduce(
        out.data_ptr(), ws_ptr, ws_bytes, context_lens.data_ptr(), int(max_context_len),
        B, Hq, D, int(partition_size), int(window), _dt(out), _stream()))


def alloc_workspace(num_seqs, num_heads, head_dim, max_context_len, partition_size,
                    device) -> Optional[torch.Tensor]:
    n = workspace_size(num_seqs, num_heads, head_dim, max_context_len, partition_size)
    if n == 0:
        return None
    return torch.empty((n + 3) // 4, dtype=torch.float32, device=device)


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, softcap=0.0, window=0,
           partition_size=None, max_context_len=None, out=None, workspace=None):
    """Paged decode attention: out[b, h] = softmax over the attended keys of
    sequence b of (capped) scale * q[b, h] . k, applied to the values.

    q [B, Hq, D]; k_cache/v_cache [NB, bs, Hkv, D]; block_tables int32
    [B, max_blocks]; context_lens int32 [B] (counting the new token).
    ``max_context_len`` defaults to context_lens.max() (one device sync).
    """
    B, Hq, D, NB, bs, Hkv = _shapes(q, k_cache, block_tables)
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if B else 0
    if partition_size is None:
        partition_size = globals()["partition_size"](B, Hq, Hkv, D, bs, max_context_len,
                                                     window, q.dtype)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = alloc_workspace(B, Hq, D, max_context_len, partition_size, q.device)
    decode_partitions(out, workspace, q, k_cache, v_cache, block_tables, context_lens,
                      max_context_len, scale, softcap, window, partition_size)
    decode_reduce(out, workspace, context_lens, max_context_len, partition_size, window)
    return out


def mq_partition_size(num_seqs, num_tokens, max_query_len, num_heads, num_kv_heads, head_dim,
                      block_size, max_context_len, window=0, dtype=torch.bfloat16) -> int:
    """The library's choice of split-K partition size for a multi-query shape."""
    return int(_lib.load().pa_mq_partition_size(
        num_seqs, num_tokens, max_query_len, num_heads, num_kv_heads, head_dim, block_size,
        max_context_len, window, _DTYPE[dtype]))


def mq_workspace_size(num_seqs, num_tokens, num_heads, num_kv_heads, head_dim, max_context_len,
                      partition_size) -> int:
    return int(_lib.load().pa_mq_workspace_size(num_seqs, num_tokens, num_heads, num_kv_heads,
                                                head_dim, max_context_len, partition_size))


def mq_attention(q, query_start, k_cache, v_cache, block_tables, context_lens, scale, softcap=0.0,
                 window=0, partition_size=None, max_context_len=None, max_query_len=None,
                 out=None, workspace=None, key=None, value=None, slot_mapping=None):
    """Multi-query paged attention (pa_mq_attention): sequence b's new tokens
    are q's rows query_start[b] .. query_start[b+1]-1, the last n_b of its
    context_lens[b] positions, each attending causally to the keys up to its
    own position.

    q [T, Hq, D]; query_start int32 [B+1]; context_lens int32 [B] (counting
    the new tokens, whose K/V rows are already in the cache).
    ``max_context_len`` / ``max_query_len`` default to the maxima of the
    device arrays (one device sync each).
    With ``key``/``value`` ([N, Hkv, D]) and ``slot_mapping`` (int64 [N]),
    the call first writes those rows into the caches as reshape_and_cache
    does, in the same launch as the plan (pa_mq_step)."""
    _dev(q, query_start, k_cache, v_cache, block_tables, context_lens, out, key, value,
         slot_mapping)
    T, Hq, D = q.shape
    NB, bs, Hkv, D2 = k_cache.shape
    B = context_lens.shape[0]
    if D2 != D:
        raise ValueError("head_dim of q and caches differ")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [num_seqs, max_blocks_per_seq]")
    if context_lens.dtype != torch.int32 or context_lens.dim() != 1:
        raise ValueError("context_lens must be int32 [num_seqs]")
    if query_start.dtype != torch.int32 or tuple(query_start.shape) != (B + 1,):
        raise ValueError("query_start must be int32 [num_seqs + 1]")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("q and caches must share a dtype")
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if B else 0
    if max_query_len is None:
        max_query_len = int((query_start[1:] - query_start[:-1]).max().item()) if B else 0
    max_query_len = max(1, min(int(max_query_len), T)) if T else 0
    if partition_size is None:
        partition_size = mq_partition_size(B, T, max(max_query_len, 1), Hq, Hkv, D, bs,
                                           max_context_len, window, q.dtype)
    if out is None:
        out = torch.empty_like(q)
    elif out.dtype != q.dtype or tuple(out.shape) != (T, Hq, D):
        raise ValueError("out must match q")
    if workspace is None:
        n = mq_workspace_size(B, T, Hq, Hkv, D, max_context_len, partition_size)
        workspace = torch.empty((n + 3) // 4, dtype=torch.float32, device=q.device) if n else None
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if slot_mapping is not None:
        a = _mq_step_args(q, query_start, k_cache, v_cache, block_tables, context_lens, scale,
                          softcap, window, partition_size, max_context_len, max_query_len, out,
                          workspace, key, value, slot_mapping)
        _lib.check("pa_mq_step", _lib.load().pa_mq_step(ctypes.byref(a), _stream()))
        return out
    if key is not None or value is not None:
        raise ValueError("key/value need slot_mapping")
    _lib.check("pa_mq_attention", _lib.load().pa_mq_attention(
        out.data_ptr(), ws_ptr, ws_bytes, q.data_ptr(), query_start.data_ptr(), T,
        int(max_query_len), k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(),
        block_tables.shape[1], context_lens.data_ptr(), int(max_context_len), B, Hq, Hkv, D, bs,
        NB, float(scale), float(softcap), int(window), int(partition_size), _dt(q), _stream()))
    return out


def _mq_step_args(q, query_start, k_cache, v_cache, block_tables, context_lens, scale, softcap,
                  window, partition_size, max_context_len, max_query_len, out, workspace, key,
                  value, slot_mapping):
    """pa_mq_step_args for checked tensors (sizes as mq_attention resolved them)."""
    T, Hq, D = q.shape
    NB, bs, Hkv, _ = k_cache.shape
    B = context_lens.shape[0]
    if slot_mapping.dtype != torch.int64 or slot_mapping.dim() != 1:
        raise TypeError("slot_mapping must be int64 [N]")
    N = slot_mapping.shape[0]
    if key is None or value is None or tuple(key.shape) != (N, Hkv, D) \
            or tuple(value.shape) != (N, Hkv, D):
        raise ValueError("key/value must be [N, Hkv, D] beside slot_mapping [N]")
    if not (key.dtype == value.dtype == q.dtype):
        raise TypeError("key, value and caches must share a dtype")
    a = _lib.MQStepArgs()
    a.key, a.value, a.slot_mapping = key.data_ptr(), value.data_ptr(), slot_mapping.data_ptr()
    a.num_new_rows = N
    a.out, a.q = out.data_ptr(), q.data_ptr()
    a.workspace = workspace.data_ptr() if workspace is not None else None
    a.workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    a.query_start, a.num_tokens, a.max_query_len = query_start.data_ptr(), T, int(max_query_len)
    a.k_cache, a.v_cache = k_cache.data_ptr(), v_cache.data_ptr()
    a.block_tables, a.max_blocks_per_seq = block_tables.data_ptr(), block_tables.shape[1]
    a.context_lens, a.max_context_len = context_lens.data_ptr(), int(max_context_len)
    a.num_seqs, a.num_heads, a.num_kv_heads, a.head_dim = B, Hq, Hkv, D
    a.block_size, a.num_blocks = bs, NB
    a.scale, a.softcap, a.window = float(scale), float(softcap), int(window)
    a.partition_size, a.dtype = int(partition_size), _dt(q)
    return a


class MQStep:
    """One multi-query layer-step over fixed buffers (pa_mq_step): the new
    K/V rows written into their slots and the new tokens' attention, built
    once (sizes resolved, output and workspace allocated) and enqueued by
    ``run`` with one native call.  Buffer contents may change between runs;
    the tensors and the host-side sizes are fixed at construction."""

    def __init__(self, q, query_start, k_cache, v_cache, block_tables, context_lens, scale,
                 softcap=0.0, window=0, partition_size=None, max_context_len=None,
                 max_query_len=None, out=None, key=None, value=None, slot_mapping=None):
        _dev(q, query_start, k_cache, v_cache, block_tables, context_lens, out, key, value,
             slot_mapping)
        T, Hq, D = q.shape
        NB, bs, Hkv, _ = k_cache.shape
        B = context_lens.shape[0]
        if max_context_len is None:
            max_context_len = int(context_lens.max().item()) if B else 0
        if max_query_len is None:
            max_query_len = int((query_start[1:] - query_start[:-1]).max().item()) if B else 0
        max_query_len = max(1, min(int(max_query_len), T)) if T else 0
        if partition_size is None:
            partition_size = mq_partition_size(B, T, max(max_query_len, 1), Hq, Hkv, D, bs,
                                               max_context_len, window, q.dtype)
        self.out = torch.empty_like(q) if out is None else out
        n = mq_workspace_size(B, T, Hq, Hkv, D, max_context_len, partition_size)
        self.workspace = (torch.empty((n + 3) // 4, dtype=torch.float32, device=q.device)
                          if n else None)
        if slot_mapping is None:  # no new rows
            slot_mapping = torch.empty(0, dtype=torch.int64, device=q.device)
            key = value = torch.empty((0, Hkv, D), dtype=q.dtype, device=q.device)
        self.args = _mq_step_args(q, query_start, k_cache, v_cache, block_tables, context_lens,
                                  scale, softcap, window, partition_size, max_context_len,
                                  max_query_len, self.out, self.workspace, key, value,
                                  slot_mapping)
        self.partition_size = int(partition_size)
        # keep every buffer alive as long as the step exists
        self._keep = (q, query_start, k_cache, v_cache, block_tables, context_lens, key, value,
                      slot_mapping, self.out, self.workspace)

    def run(self):
        """Enqueue the step on torch's current stream."""
        _lib.check("pa_mq_step", _lib.load().pa_mq_step(ctypes.byref(self.args), _stream()))
        return self.out


class Step:
    """One layer-step over fixed buffers: reshape_and_cache of the new rows
    (if given), pa_decode and pa_decode_reduce, run through pa_step, or
    captured once into a HIP graph (``capture``) and replayed with
    ``replay``.  Buffer contents may change between runs; the tensors (and
    so their addresses) and the host-side sizes are fixed at construction.
    ``rows_at_tails``: key/value/slot_mapping have one row per sequence, row
    i being sequence i's newest token (slot -1: none), so the decode launch
    writes them itself."""

    def __init__(self, q, k_cache, v_cache, block_tables, context_lens, scale, softcap=0.0,
                 window=0, partition_size=None, max_context_len=None, out=None,
                 key=None, value=None, slot_mapping=None, rows_at_tails=False):
        B, Hq, D, NB, bs, Hkv = _shapes(q, k_cache, block_tables)
        _dev(q, k_cache, v_cache, block_tables, context_lens, key, value, slot_mapping)
        if max_context_len is None:
            max_context_len = int(context_lens.max().item()) if B else 0
        if partition_size is None:
            partition_size = globals()["partition_size"](B, Hq, Hkv, D, bs, max_context_len,
                                                         window, q.dtype)
        self.out = torch.empty_like(q) if out is None else out
        self.workspace = alloc_workspace(B, Hq, D, max_context_len, partition_size, q.device)
        # keep every buffer alive as long as the step (and its graph) exists
        self._keep = (q, k_cache, v_cache, block_tables, context_lens, key, value,
                      slot_mapping, self.out, self.workspace)
        a = _lib.StepArgs()
        if slot_mapping is not None:
            a.key, a.value, a.slot_mapping = key.data_ptr(), value.data_ptr(), slot_mapping.data_ptr()
            a.num_tokens = slot_mapping.shape[0]
        a.out, a.q = self.out.data_ptr(), q.data_ptr()
        a.workspace = self.workspace.data_ptr() if self.workspace is not None else None
        a.workspace_bytes = (self.workspace.numel() * 4) if self.workspace is not None else 0
        a.k_cache, a.v_cache = k_cache.data_ptr(), v_cache.data_ptr()
        a.block_tables, a.max_blocks_per_seq = block_tables.data_ptr(), block_tables.shape[1]
        a.context_lens, a.max_context_len = context_lens.data_ptr(), int(max_context_len)
        a.num_seqs, a.num_heads, a.num_kv_heads, a.head_dim = B, Hq, Hkv, D
        a.block_size, a.num_blocks = bs, NB
        a.scale, a.softcap, a.window = float(scale), float(softcap), int(window)
        a.partition_size, a.dtype = int(partition_size), _dt(q)
        # row i of key/value is sequence i's newest token (a decode step)
        a.new_rows_at_tails = 1 if rows_at_tails else 0
        self.args = a
        self.partition_size = int(partition_size)
        self._graph = None

    def run(self):
        """Enqueue the step on torch's current stream."""
        _lib.check("pa_step", _lib.load().pa_step(ctypes.byref(self.args), _stream()))
        return self.out

    def run_static(self):
        """Enqueue the step through pa_step_static (scratch in the library's
        static per-GPU array; this object's workspace is not used)."""
        _lib.check("pa_step_static",
                   _lib.load().pa_step_static(ctypes.byref(self.args), _stream()))
        return self.out

    def capture(self, stream):
        """Capture the step on ``stream`` (a torch.cuda.Stream, not the
        default stream) into a HIP graph."""
        self.close()
        h = ctypes.c_void_p()
        _lib.check("pa_step_graph_create", _lib.load().pa_step_graph_create(
            ctypes.byref(self.args), stream.cuda_stream, ctypes.byref(h)))
        self._graph = h
        return self

    def replay(self, stream=None):
        """Enqueue one replay of the captured step (on ``stream`` or torch's
        current stream)."""
        if self._graph is None:
            raise RuntimeError("capture() first")
        s = (stream or torch.cuda.current_stream()).cuda_stream
        _lib.check("pa_step_graph_launch", _lib.load().pa_step_graph_launch(self._graph, s))
        return self.out

    def close(self):
        if self._graph is not None:
            _lib.load().pa_step_graph_destroy(self._graph)
            self._graph = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class StepGraph:
    """Several layer steps (Step objects, e.g. one per layer of a model)
    captured into one HIP graph on ``stream`` (a torch.cuda.Stream) and
    replayed by one launch, in the order given (pa_step_graph_create_n)."""

    def __init__(self, steps, stream):
        if not steps:
            raise ValueError("no steps")
        self.steps = list(steps)
        arr = (_lib.StepArgs * len(self.steps))(*[st.args for st in self.steps])
        self._arr = arr
        h = ctypes.c_void_p()
        _lib.check("pa_step_graph_create_n", _lib.load().pa_step_graph_create_n(
            arr, len(self.steps), stream.cuda_stream, ctypes.byref(h)))
        self._graph = h

    def replay(self, stream=None):
        """Enqueue one replay of every captured step (on ``stream`` or
        torch's current stream)."""
        if self._graph is None:
            raise RuntimeError("graph closed")
        s = (stream or torch.cuda.current_stream()).cuda_stream
        _lib.check("pa_step_graph_launch", _lib.load().pa_step_graph_launch(self._graph, s))

    def close(self):
        if self._graph is not None:
            _lib.load().pa_step_graph_destroy(self._graph)
            self._graph = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
