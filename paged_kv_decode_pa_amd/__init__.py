"""Paged KV-cache decode attention for AMD MI355X (gfx950).

Hand-written HIP kernels behind a C ABI (include/pa.h, libpa.so); this
package is a thin binding that marshals torch tensors (device memory) and
torch's current stream into those calls.
"""
from ._lib import EXPORTS, LIB_PATH, PaError, load, status_string
from .ops import (MQStep, Step, StepGraph, alloc_workspace, copy_blocks, decode, decode_partitions,
                  decode_reduce, mq_attention, mq_partition_size, mq_workspace_size,
                  partition_size, read_bandwidth_probe, reshape_and_cache, set_decode_events,
                  workspace_size)

__all__ = ["EXPORTS", "LIB_PATH", "MQStep", "PaError", "Step", "StepGraph", "load", "status_string",
           "alloc_workspace", "copy_blocks", "mq_attention", "mq_partition_size", "mq_workspace_size",
           "decode", "decode_partitions", "decode_reduce", "partition_size",
           "read_bandwidth_probe", "reshape_and_cache", "set_decode_events", "workspace_size"]
