"""pa_step against the float64 oracle on the launch shapes its preparation
launch (new K/V rows and the sequence plan in one launch) meets: the vector
and matrix-core kernels, one workgroup per unit and looping launches, with
and without the plan, with and without new rows, split and unsplit keys.
Each step runs twice on the same buffers, and pa_step must equal the three
separate calls (PA_STEP_FUSE=0) bit for bit.

Tolerance as for pa_decode: 1e-4 for float32 KV, 2e-2 for 16-bit KV."""
import os

import numpy as np
import pytest

import oracle
from workloads import make_case

pytestmark = pytest.mark.gpu


def _lens(rng, B, lo, hi, extra=()):
    L = list(rng.integers(lo, hi, size=B - len(extra), endpoint=True)) + list(extra)
    return [int(x) for x in L]


# name, dtype, Hq, Hkv, D, bs, softcap, window, P, B, (lo, hi), extra lengths, new rows, env
CASES = [
    # vector kernel, 64 sequences (plan in the preparation launch), 8 partitions
    ("valu-plan", "bf16", 8, 4, 256, 16, 50.0, 0, 128, 64, (128, 1024), (0, 1, 128, 129), True, {}),
    # vector kernel, 16 sequences, sliding window, 16 partitions, XCD-grouped grid
    ("valu-window", "bf16", 8, 4, 256, 16, 50.0, 300, 64, 16, (400, 1024), (1, 64), True, {}),
    # vector kernel, looping launch over the plan's items
    ("valu-loop", "bf16", 8, 4, 128, 16, 0.0, 0, 64, 200, (700, 1024), (0, 65), True, {}),
    # float32 vector kernel, no new rows, no plan: no preparation launch
    ("valu-f32-norows", "f32", 8, 2, 64, 16, 0.0, 0, 32, 9, (1, 500), (0, 1, 33), False, {}),
    # matrix cores, one wavefront per KV head, 16 partitions
    ("mfma-heads", "f16", 32, 4, 64, 32, 0.0, 0, 128, 6, (1, 2048), (0, 1, 2048), True, {}),
    # matrix cores, per-head workgroups (heads mode off)
    ("mfma-split", "bf16", 16, 2, 128, 32, 30.0, 0, 64, 7, (1, 1000), (0, 999), True,
     {"PA_DECODE_HEADS": "0"}),
    # matrix cores, heads mode, looping launch
    ("mfma-heads-loop", "f16", 32, 4, 64, 32, 0.0, 0, 64, 200, (600, 1024), (0, 1), True, {}),
    # many partitions
    ("mfma-reduce", "f16", 32, 4, 64, 32, 0.0, 0, 64, 6, (1, 2000), (0, 1, 2000), True, {}),
    ("valu-reduce", "bf16", 8, 4, 256, 16, 50.0, 0, 32, 5, (1, 1000), (0, 999), False, {}),
    # no split at all
    ("valu-nosplit", "bf16", 8, 4, 256, 16, 50.0, 0, 0, 50, (1, 600), (0,), True, {}),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_step_matches_oracle(case):
    import torch
    import paged_kv_decode_pa_amd as pa
    from gpu_util import TOL, DeviceCase, say, to_f64
    name, dt, Hq, Hkv, D, bs, cap, W, P, B, (lo, hi), extra, rows, env = case
    say(f"step {name}")
    rng = np.random.default_rng(sum(map(ord, name)))
    c = make_case(B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs, dtype=dt,
                  context_lens=_lens(rng, B, lo, hi, extra), softcap=cap, window=W,
                  partition_size=P, seed=sum(map(ord, name)) + 7, new_rows=rows,
                  extra_table_cols=2)
    want = oracle.decode_case(c)
    dc = DeviceCase(c)
    saved = {k: os.environ.get(k) for k in list(env) + ["PA_STEP_FUSE"]}
    os.environ.update(env)
    got = {}
    try:
        step = pa.Step(dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, c.scale,
                       c.softcap, c.window, partition_size=P, max_context_len=c.max_context_len,
                       key=dc.key, value=dc.value, slot_mapping=dc.slot_mapping)
        for fuse in ("1", "0"):
            os.environ["PA_STEP_FUSE"] = fuse
            first = to_f64(step.run().clone())
            torch.cuda.synchronize()
            second = to_f64(step.run().clone())
            torch.cuda.synchronize()
            assert np.array_equal(first, second), f"fuse={fuse}: second step differs"
            got[fuse] = first
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    assert np.isfinite(got["1"]).all(), "non-finite output"
    err = np.abs(got["1"] - want).max()
    assert err <= TOL[dt], f"max abs err {err:.3g} > {TOL[dt]}"
    assert np.array_equal(got["1"], got["0"]), "pa_step differs from the three calls"


def _rows_per_sequence(c):
    """The case's new rows laid out one per sequence (row i = sequence i's
    newest token; slot -1 and zero rows for empty sequences), as a decode
    step hands them over."""
    live = [b for b in range(c.B) if c.context_lens[b] > 0]
    shape = (c.B,) + c.key.shape[1:]
    key = np.zeros(shape, dtype=c.key.dtype)
    value = np.zeros(shape, dtype=c.value.dtype)
    slots = np.full(c.B, -1, dtype=np.int64)
    key[live], value[live], slots[live] = c.key, c.value, c.slot_mapping
    return key, value, slots


ROW_CASES = [cs for cs in CASES if cs[12]]


@pytest.mark.parametrize("case", ROW_CASES, ids=[c[0] for c in ROW_CASES])
def test_step_rows_at_tails(case):
    """New rows handed over one per sequence at its last position: on the
    vector kernel the decode launch writes them itself.  Output and caches
    equal the three separate calls bit for bit, twice in a row, and the
    output matches the oracle."""
    import torch
    import paged_kv_decode_pa_amd as pa
    from gpu_util import TOL, DeviceCase, say, to_f64
    name, dt, Hq, Hkv, D, bs, cap, W, P, B, (lo, hi), extra, rows, env = case
    say(f"step rows at tails {name}")
    rng = np.random.default_rng(sum(map(ord, name)) + 1)
    c = make_case(B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs, dtype=dt,
                  context_lens=_lens(rng, B, lo, hi, extra), softcap=cap, window=W,
                  partition_size=P, seed=sum(map(ord, name)) + 11, new_rows=True,
                  extra_table_cols=2)
    c.key, c.value, c.slot_mapping = _rows_per_sequence(c)
    want = oracle.decode_case(c)
    results = {}
    saved = {k: os.environ.get(k) for k in list(env) + ["PA_STEP_FUSE"]}
    os.environ.update(env)
    try:
        for fuse in ("1", "0"):
            os.environ["PA_STEP_FUSE"] = fuse
            dc = DeviceCase(c)
            step = pa.Step(dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                           c.scale, c.softcap, c.window, partition_size=P,
                           max_context_len=c.max_context_len, key=dc.key, value=dc.value,
                           slot_mapping=dc.slot_mapping, rows_at_tails=True)
            first = to_f64(step.run().clone())
            torch.cuda.synchronize()
            second = to_f64(step.run().clone())
            torch.cuda.synchronize()
            assert np.array_equal(first, second), f"fuse={fuse}: second step differs"
            bits = lambda t: t.view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu().numpy()
            results[fuse] = (first, bits(dc.k_cache), bits(dc.v_cache))
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    out, kc, vc = results["1"]
    assert np.isfinite(out).all(), "non-finite output"
    assert np.abs(out - want).max() <= TOL[dt]
    assert np.array_equal(out, results["0"][0]), "differs from the three calls"
    assert np.array_equal(kc, results["0"][1]) and np.array_equal(vc, results["0"][2]), \
        "caches differ from reshape_and_cache's"
