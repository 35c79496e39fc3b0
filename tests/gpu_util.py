"""Helpers for the GPU tests: upload a synthetic case and run the library."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
TOL = {"f32": 1e-4, "f16": 2e-2, "bf16": 2e-2}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def upload(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(TORCH_DT[dtype])
    return torch.from_numpy(a).to(device)


class DeviceCase:
    def __init__(self, case, device="cuda"):
        self.case = case
        self.q = upload(case.q, case.dtype, device)
        self.k_cache = upload(case.k_cache, case.dtype, device)
        self.v_cache = upload(case.v_cache, case.dtype, device)
        self.block_tables = torch.from_numpy(case.block_tables).to(device)
        self.context_lens = torch.from_numpy(case.context_lens).to(device)
        self.key = self.value = self.slot_mapping = None
        if case.slot_mapping is not None:
            self.key = upload(case.key, case.dtype, device)
            self.value = upload(case.value, case.dtype, device)
            self.slot_mapping = torch.from_numpy(case.slot_mapping).to(device)


def run_step(dc: DeviceCase, partition_size=None, waves=None, out=None, env=None):
    """reshape_and_cache (if the case has new rows) then decode + reduce;
    env: further library switches for this call."""
    import paged_kv_decode_pa_amd as pa
    c = dc.case
    env = dict(env or {})
    if waves is not None:
        env["PA_DECODE_WAVES"] = str(waves)
    os.environ.update(env)
    try:
        if dc.slot_mapping is not None:
            pa.reshape_and_cache(dc.key, dc.value, dc.k_cache, dc.v_cache, dc.slot_mapping)
        P = c.partition_size if partition_size is None else partition_size
        # None: the library picks the split for this shape
        out = pa.decode(dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                        c.scale, c.softcap, c.window, partition_size=P,
                        max_context_len=c.max_context_len, out=out)
        torch.cuda.synchronize()
    finally:
        for k in env:
            os.environ.pop(k, None)
    return out


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)
