"""ctypes loader for libpa.so and the raw C entry points.

The library must be built in-tree first (``python -m
paged_kv_decode_pa_amd.build``); loading fails loudly when it is missing.
There is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpa.so")

PA_F32, PA_F16, PA_BF16 = 0, 1, 2
STATUS = {0: "PA_OK", -1: "PA_EINVAL", -2: "PA_EUNSUPPORTED", -3: "PA_EWORKSPACE",
          -4: "PA_ELAUNCH", -5: "PA_ESCRATCH"}
PA_STATIC_SCRATCH_BYTES = 128 << 20

# every symbol include/pa.h declares
EXPORTS = ("pa_status_string", "pa_reshape_and_cache", "pa_decode_partition_size",
           "pa_decode_workspace_size", "pa_decode", "pa_decode_reduce", "pa_copy_blocks",
           "pa_mq_partition_size", "pa_mq_workspace_size", "pa_mq_attention", "pa_step",
           "pa_step_graph_create", "pa_step_graph_create_n", "pa_step_graph_launch",
           "pa_step_graph_destroy", "pa_step_static", "pa_set_decode_events",
           "pa_read_bandwidth_probe", "pa_mq_step")


class StepArgs(ctypes.Structure):
    """pa_step_args (include/pa.h)."""
    _fields_ = [
        ("key", ctypes.c_void_p), ("value", ctypes.c_void_p),
        ("slot_mapping", ctypes.c_void_p), ("num_tokens", ctypes.c_int),
        ("out", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t), ("q", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("block_tables", ctypes.c_void_p), ("max_blocks_per_seq", ctypes.c_int),
        ("context_lens", ctypes.c_void_p), ("max_context_len", ctypes.c_int),
        ("num_seqs", ctypes.c_int), ("num_heads", ctypes.c_int),
        ("num_kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int),
        ("block_size", ctypes.c_int), ("num_blocks", ctypes.c_int),
        ("scale", ctypes.c_float), ("softcap", ctypes.c_float), ("window", ctypes.c_int),
        ("partition_size", ctypes.c_int), ("dtype", ctypes.c_int),
        ("new_rows_at_tails", ctypes.c_int),
    ]


class MQStepArgs(ctypes.Structure):
    """pa_mq_step_args (include/pa.h)."""
    _fields_ = [
        ("key", ctypes.c_void_p), ("value", ctypes.c_void_p),
        ("slot_mapping", ctypes.c_void_p), ("num_new_rows", ctypes.c_int),
        ("out", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t), ("q", ctypes.c_void_p),
        ("query_start", ctypes.c_void_p), ("num_tokens", ctypes.c_int),
        ("max_query_len", ctypes.c_int),
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("block_tables", ctypes.c_void_p), ("max_blocks_per_seq", ctypes.c_int),
        ("context_lens", ctypes.c_void_p), ("max_context_len", ctypes.c_int),
        ("num_seqs", ctypes.c_int), ("num_heads", ctypes.c_int),
        ("num_kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int),
        ("block_size", ctypes.c_int), ("num_blocks", ctypes.c_int),
        ("scale", ctypes.c_float), ("softcap", ctypes.c_float), ("window", ctypes.c_int),
        ("partition_size", ctypes.c_int), ("dtype", ctypes.c_int),
    ]


_lib = None


class PaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({status_string(status)})")


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m paged_kv_decode_pa_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64p, sz, f32 = (ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                             ctypes.c_size_t, ctypes.c_float)
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_status_string.argtypes = [i32]
    lib.pa_reshape_and_cache.restype = i32
    lib.pa_reshape_and_cache.argtypes = [vp, vp, vp, vp, i64p, i32, i32, i32, i32, i32, i32, vp]
    lib.pa_decode_partition_size.restype = i32
    lib.pa_decode_partition_size.argtypes = [i32] * 8
    lib.pa_decode_workspace_size.restype = sz
    lib.pa_decode_workspace_size.argtypes = [i32] * 5
    lib.pa_decode.restype = i32
    lib.pa_decode.argtypes = [vp, vp, sz, vp, vp, vp, vp, i32, vp, i32,
                              i32, i32, i32, i32, i32, i32, f32, f32, i32, i32, i32, vp]
    lib.pa_decode_reduce.restype = i32
    lib.pa_decode_reduce.argtypes = [vp, vp, sz, vp, i32, i32, i32, i32, i32, i32, i32, vp]
    lib.pa_copy_blocks.restype = i32
    lib.pa_copy_blocks.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    lib.pa_mq_partition_size.restype = i32
    lib.pa_mq_partition_size.argtypes = [i32] * 10
    lib.pa_mq_workspace_size.restype = sz
    lib.pa_mq_workspace_size.argtypes = [i32] * 7
    lib.pa_mq_attention.restype = i32
    lib.pa_mq_attention.argtypes = [vp, vp, sz, vp, vp, i32, i32, vp, vp, vp, i32, vp, i32,
                                    i32, i32, i32, i32, i32, i32, f32, f32, i32, i32, i32, vp]
    sp = ctypes.POINTER(StepArgs)
    lib.pa_step.restype = i32
    lib.pa_step.argtypes = [sp, vp]
    lib.pa_step_graph_create.restype = i32
    lib.pa_step_graph_create.argtypes = [sp, vp, ctypes.POINTER(ctypes.c_void_p)]
    lib.pa_step_graph_create_n.restype = i32
    lib.pa_step_graph_create_n.argtypes = [sp, i32, vp, ctypes.POINTER(ctypes.c_void_p)]
    lib.pa_step_graph_launch.restype = i32
    lib.pa_step_graph_launch.argtypes = [vp, vp]
    lib.pa_step_graph_destroy.restype = i32
    lib.pa_step_graph_destroy.argtypes = [vp]
    lib.pa_step_static.restype = i32
    lib.pa_step_static.argtypes = [sp, vp]
    lib.pa_set_decode_events.restype = i32
    lib.pa_set_decode_events.argtypes = [vp, vp]
    lib.pa_mq_step.restype = i32
    lib.pa_mq_step.argtypes = [ctypes.POINTER(MQStepArgs), vp]
    lib.pa_read_bandwidth_probe.restype = i32
    lib.pa_read_bandwidth_probe.argtypes = [vp, sz, i32, vp, vp]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().pa_status_string(status).decode()


def check(fn: str, status: int) -> None:
    if status != 0:
        raise PaError(fn, status)
