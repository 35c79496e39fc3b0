"""Decode attention on the GPU against the float64 oracle, element by element.

Tolerance (max abs error): 1e-4 for float32 KV, 2e-2 for float16/bfloat16 KV
(float32 accumulation, output rounded to the storage type).  Unreferenced
blocks, the unused tail of every last block and block-table padding hold NaN
or -1, so any read outside the attended keys poisons the result."""
import numpy as np
import pytest

import oracle
from workloads import gather_logical, assign_blocks, layout_cache, make_case, workload

pytestmark = pytest.mark.gpu


def gpu(case, **kw):
    from gpu_util import DeviceCase, run_step, to_f64
    return to_f64(run_step(DeviceCase(case), **kw))


def check(case, got, seqs=None, tol=None, want=None):
    """Compare the rows of ``seqs`` (all when None) with the oracle; every
    output row, compared or not, must be finite (a read of a NaN-poisoned
    slot anywhere shows up here)."""
    from gpu_util import TOL
    tol = TOL[case.dtype] if tol is None else tol
    assert np.isfinite(got).all(), "non-finite output"
    if want is None:
        want = oracle.decode_case(case, seqs=seqs)
    rows = slice(None) if seqs is None else list(seqs)
    err = np.abs(got[rows] - want[rows])
    assert err.max() <= tol, f"max abs err {err.max():.3g} > {tol}"
    return float(err.max())


_ORACLE = {}


def oracle_workload(n):
    """The oracle's output for every sequence of workload n (computed once
    per test session: a few seconds for the largest)."""
    if n not in _ORACLE:
        _ORACLE[n] = oracle.decode_case(workload(n))
    return _ORACLE[n]


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------
def test_workload1_tiny_f32():
    from gpu_util import say
    say("workload 1")
    c = workload(1)
    for waves in (None, 1, 2, 4, 8):
        check(c, gpu(c, waves=waves))


@pytest.mark.parametrize("P", [None, 0, 128, 512])
def test_workload2_gemma_global_with_new_rows(P):
    from gpu_util import say
    say(f"workload 2 P={P}")
    c = workload(2)
    check(c, gpu(c, partition_size=P))
    if P is None:  # the default launch runs without a plan; with one too
        check(c, gpu(c, env={"PA_DECODE_PLAN": "1"}))


def test_workload2_step_rows_at_tails():
    """The global-layer step as bench.py runs it: pa_step with the new rows
    handed over one per sequence, written by the decode launch itself (no
    preparation launch).  Every sequence against the oracle; the caches
    equal reshape_and_cache's bit for bit."""
    import torch
    import paged_kv_decode_pa_amd as pa
    from gpu_util import DeviceCase, say, to_f64
    say("workload 2 step, rows at tails")
    c = workload(2)
    assert c.slot_mapping.shape[0] == c.B
    dc = DeviceCase(c)
    st = pa.Step(dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, c.scale,
                 c.softcap, c.window, max_context_len=c.max_context_len, key=dc.key,
                 value=dc.value, slot_mapping=dc.slot_mapping, rows_at_tails=True)
    check(c, to_f64(st.run()), want=oracle_workload(2))
    wk, wv = oracle.reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping)
    back = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    assert back(dc.k_cache).tobytes() == wk.tobytes()
    assert back(dc.v_cache).tobytes() == wv.tobytes()


def test_workload3_gemma_sliding_window():
    """The default launch here is the whole grid resident as two-wavefront
    workgroups with wave priority; eight-wavefront workgroups (no priority)
    must agree with the oracle too, and priority on or off changes only the
    schedule: identical bits."""
    import os
    from gpu_util import say
    say("workload 3")
    c = workload(3)
    got = gpu(c)
    check(c, got)
    check(c, gpu(c, waves=8))
    os.environ["PA_DECODE_PRIO"] = "0"
    try:
        same = gpu(c)
    finally:
        os.environ.pop("PA_DECODE_PRIO", None)
    assert np.array_equal(got, same)


@pytest.mark.parametrize("P", [None, 0, 256])
def test_workload4_serving_b512(P):
    from gpu_util import say
    say(f"workload 4 P={P}")
    c = workload(4)
    got = gpu(c, partition_size=P)
    check(c, got, want=oracle_workload(4))


def test_workload5_llama_long_context():
    from gpu_util import say
    say("workload 5")
    c = workload(5)
    got = gpu(c)
    check(c, got, want=oracle_workload(5))


# --------------------------------------------------------------------------
# a matrix of small shapes: several chunks, ragged tails, every dtype
# --------------------------------------------------------------------------
SHAPES = [
    # dtype, Hq, Hkv, D, bs, softcap, window, P
    ("f32", 8, 2, 64, 16, 0.0, 0, 0),
    ("f32", 4, 4, 128, 8, 30.0, 0, 64),
    ("f32", 16, 2, 256, 32, 0.0, 50, 32),
    ("f16", 32, 4, 64, 32, 0.0, 0, 64),
    ("f16", 8, 8, 128, 16, 50.0, 70, 0),
    ("f16", 16, 4, 256, 1, 0.0, 0, 48),
    ("bf16", 8, 4, 256, 16, 50.0, 0, 0),
    ("bf16", 8, 4, 256, 16, 50.0, 0, 64),
    ("bf16", 8, 2, 128, 2, 20.0, 33, 16),
    ("bf16", 32, 4, 64, 32, 0.0, 0, 32),
    ("bf16", 32, 8, 128, 64, 0.0, 100, 128),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[0]}-g{s[1]//s[2]}-d{s[3]}-bs{s[4]}-c{s[5]:g}-w{s[6]}-p{s[7]}" for s in SHAPES])
@pytest.mark.parametrize("waves", [None, 1, 4, 8])
def test_small_shapes(shape, waves):
    from gpu_util import say
    dt, Hq, Hkv, D, bs, cap, W, P = shape
    say(f"small {shape} waves={waves}")
    L = [1, 2, 17, 100, 255, 513, 64, 31]
    c = make_case(B=len(L), Hq=Hq, Hkv=Hkv, D=D, bs=bs, dtype=dt, context_lens=L,
                  softcap=cap, window=W, partition_size=P, seed=sum(map(ord, str(shape))),
                  extra_table_cols=3)
    check(c, gpu(c, waves=waves))


# --------------------------------------------------------------------------
# the matrix-core path (groups of 8 or 16 query heads, 16-bit KV, pages of
# 16+ tokens) against the oracle, and the vector path on the same shapes
# --------------------------------------------------------------------------
MFMA_SHAPES = [
    # dtype, Hq, Hkv, D, bs, softcap, window, P
    ("f16", 32, 4, 64, 32, 0.0, 0, 512),
    ("f16", 32, 4, 64, 16, 0.0, 0, 0),
    ("bf16", 16, 2, 128, 32, 50.0, 0, 64),
    ("bf16", 8, 1, 256, 16, 30.0, 45, 32),
    ("f16", 32, 2, 128, 32, 0.0, 0, 96),
    ("bf16", 64, 4, 64, 64, 50.0, 100, 0),
    ("f16", 16, 1, 256, 32, 0.0, 0, 0),
]


# path -> environment: the matrix-core kernel with one wavefront per KV head
# (default) or with wavefronts splitting one head's chunks, and the vector
# kernel with and without the XCD-grouped grid
GROUP_PATHS = {
    "mfma-heads": {"PA_DECODE_MFMA": "1", "PA_DECODE_HEADS": "1"},
    "mfma-split": {"PA_DECODE_MFMA": "1", "PA_DECODE_HEADS": "0"},
    "valu-xcd": {"PA_DECODE_MFMA": "0", "PA_DECODE_XCD": "1"},
    "valu-plain": {"PA_DECODE_MFMA": "0", "PA_DECODE_XCD": "0"},
}


@pytest.mark.parametrize("shape", MFMA_SHAPES,
                         ids=[f"{s[0]}-g{s[1]//s[2]}-d{s[3]}-bs{s[4]}-c{s[5]:g}-w{s[6]}-p{s[7]}" for s in MFMA_SHAPES])
@pytest.mark.parametrize("path", list(GROUP_PATHS))
def test_group_path_shapes(shape, path):
    import os
    from gpu_util import say
    dt, Hq, Hkv, D, bs, cap, W, P = shape
    G = Hq // Hkv
    if path.startswith("valu") and G > 8:
        pytest.skip("the vector path takes groups of up to 8 heads")
    say(f"group path {path} {shape}")
    L = [1, 5, 33, 200, 700, 64, 1000]
    c = make_case(B=len(L), Hq=Hq, Hkv=Hkv, D=D, bs=bs, dtype=dt, context_lens=L,
                  softcap=cap, window=W, partition_size=P, seed=sum(map(ord, str(shape))) + 7,
                  extra_table_cols=2)
    env = GROUP_PATHS[path]
    os.environ.update(env)
    try:
        for waves in (1, 4):
            check(c, gpu(c, waves=waves))
    finally:
        for k in env:
            os.environ.pop(k, None)


def test_looping_launch_over_many_partitions():
    """One long sequence among short ones with small partitions: the grid of
    every (sequence, KV head, partition) would be mostly empty, so the launch
    loops over the plan's list of non-empty partitions instead."""
    import paged_kv_decode_pa_amd as pa
    from gpu_util import say
    say("looping launch")
    rng = np.random.default_rng(12)
    L = [8192] + list(rng.integers(1, 300, size=39))
    c = make_case(B=40, Hq=8, Hkv=4, D=128, bs=16, dtype="bf16", context_lens=L,
                  softcap=50.0, partition_size=64, seed=13)
    NP = -(-8192 // 64)
    assert 40 * 4 * NP > 2 * 256 * 16  # more workgroups than the heuristic allows
    check(c, gpu(c))
    c5 = make_case(B=40, Hq=32, Hkv=4, D=64, bs=32, dtype="f16", context_lens=L,
                   partition_size=64, seed=14)
    check(c5, gpu(c5))


# --------------------------------------------------------------------------
# invariants and edge cases on the GPU
# --------------------------------------------------------------------------
def test_single_key_is_exact():
    from gpu_util import say
    say("single key")
    c = make_case(B=5, Hq=8, Hkv=4, D=256, bs=16, dtype="bf16", context_lens=[1] * 5,
                  softcap=50.0, seed=3)
    got = gpu(c)
    want = oracle.decode_case(c)
    assert np.array_equal(got, want)


def test_window_one_is_exact():
    from gpu_util import say
    say("window one")
    c = make_case(B=4, Hq=8, Hkv=2, D=128, bs=16, dtype="f16", context_lens=[3, 40, 200, 1000],
                  window=1, seed=4, partition_size=64)
    assert np.array_equal(gpu(c), oracle.decode_case(c))


def test_empty_sequences_give_zero():
    from gpu_util import say
    say("empty sequences")
    c = make_case(B=4, Hq=8, Hkv=4, D=64, bs=16, dtype="bf16", context_lens=[0, 30, 0, 600],
                  seed=5, partition_size=128)
    got = gpu(c)
    assert np.all(got[[0, 2]] == 0)
    check(c, got)


def test_block_permutation_is_bit_identical():
    from gpu_util import say
    say("block permutation")
    c = make_case(B=6, Hq=8, Hkv=4, D=256, bs=16, dtype="bf16",
                  context_lens=[5, 77, 160, 300, 511, 1024], softcap=50.0, seed=6,
                  partition_size=256)
    a = gpu(c)
    perm = np.random.default_rng(1).permutation(c.NB)
    kc, vc = np.empty_like(c.k_cache), np.empty_like(c.v_cache)
    kc[perm], vc[perm] = c.k_cache, c.v_cache
    c.block_tables = np.where(c.block_tables >= 0, perm[np.maximum(c.block_tables, 0)],
                              -1).astype(np.int32)
    c.k_cache, c.v_cache = kc, vc
    assert np.array_equal(gpu(c), a)


def test_block_size_one_vs_sixteen():
    from gpu_util import say
    say("block size 1 vs 16")
    c16 = make_case(B=3, Hq=8, Hkv=2, D=128, bs=16, dtype="bf16", context_lens=[9, 130, 400],
                    softcap=50.0, seed=8, partition_size=0)
    lk = gather_logical(c16.k_cache, c16.block_tables, c16.context_lens)
    lv = gather_logical(c16.v_cache, c16.block_tables, c16.context_lens)
    NB = sum(int(x) for x in c16.context_lens) + 3
    bt = assign_blocks(c16.context_lens, 1, NB, np.random.default_rng(2))
    c1 = make_case(B=3, Hq=8, Hkv=2, D=128, bs=1, dtype="bf16", context_lens=[9, 130, 400],
                   softcap=50.0, seed=8, partition_size=0, NB=NB)
    c1.q = c16.q
    c1.block_tables = bt
    c1.k_cache = layout_cache(lk, bt, NB, 1, "bf16")
    c1.v_cache = layout_cache(lv, bt, NB, 1, "bf16")
    a, b = gpu(c16), gpu(c1)
    assert np.abs(a - b).max() <= 2e-2
    check(c1, b)


def test_gqa_head_map():
    from gpu_util import say
    say("gqa map")
    c = make_case(B=3, Hq=32, Hkv=4, D=64, bs=32, dtype="f16", context_lens=[10, 99, 700],
                  seed=9, partition_size=128)
    for g in range(c.Hkv):
        c.v_cache[:, :, g, :] = np.float16(g + 1).view(np.uint16)
    got = gpu(c)
    for h in range(c.Hq):
        assert np.all(got[:, h, :] == h // 8 + 1)


def test_decode_events_bracket_the_decode_kernel():
    """With the event hook set, pa_decode records the events around its
    decode kernel only: a positive time no longer than the whole call's
    (plan launch included), and the same output bits as without it."""
    import torch
    import paged_kv_decode_pa_amd as pa
    from gpu_util import DeviceCase, run_step, say, to_f64
    say("decode events")
    L = list(range(1, 1000, 17))  # 59 sequences: the plan runs before the decode kernel
    c = make_case(B=len(L), Hq=8, Hkv=4, D=256, bs=16, dtype="bf16", context_lens=L,
                  softcap=50.0, seed=44, partition_size=0)
    dc = DeviceCase(c)
    ref = to_f64(run_step(dc))
    s = torch.cuda.current_stream()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for x in e[:2]:
        x.record(s)
    pa.set_decode_events(e[0], e[1])
    try:
        e[2].record(s)
        got = run_step(dc)
        e[3].record(s)
    finally:
        pa.set_decode_events()
    torch.cuda.synchronize()
    kern, call = e[0].elapsed_time(e[1]), e[2].elapsed_time(e[3])
    assert 0.0 < kern <= call
    assert np.array_equal(to_f64(got), ref)
    check(c, ref)


def test_output_guard_band_untouched():
    import torch
    from gpu_util import DeviceCase, run_step, say
    say("guard band")
    c = make_case(B=4, Hq=8, Hkv=4, D=256, bs=16, dtype="bf16", context_lens=[3, 60, 700, 1],
                  seed=10, partition_size=128)
    big = torch.full((c.B + 2, c.Hq, c.D), 7.0, dtype=torch.bfloat16, device="cuda")
    out = big[1:1 + c.B]
    run_step(DeviceCase(c), out=out)
    assert torch.all(big[0] == 7.0) and torch.all(big[-1] == 7.0)
    check(c, out.float().cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("P", [0, 16])
def test_many_sequences(P):
    """More sequences than one plan slice (1,024), mixed lengths (the plan's
    order and, with a split, its item list)."""
    from gpu_util import say
    say(f"many sequences P={P}")
    rng = np.random.default_rng(91)
    B = 3000
    L = rng.integers(0, 60, size=B)
    c = make_case(B=B, Hq=8, Hkv=2, D=64, bs=16, dtype="f16", context_lens=L, seed=92,
                  partition_size=P, poison=False)
    check(c, gpu(c))


# --------------------------------------------------------------------------
# maximum sizes: KV pools past 4 GiB (64-bit page offsets) and the largest
# block size
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dt,Hq,Hkv,D,bs,cap,P", [
    ("bf16", 8, 4, 256, 16, 50.0, 256),   # vector kernel
    ("f16", 32, 4, 64, 32, 0.0, 512),     # matrix-core kernel
])
def test_pool_beyond_4gib(dt, Hq, Hkv, D, bs, cap, P):
    """A small case whose pages sit at the top of K and V pools of more than
    4 GiB each (built on the GPU, NaN everywhere else): page offsets past
    2^32 bytes, for decode and for a new row written by reshape_and_cache."""
    import torch
    import paged_kv_decode_pa_amd as pa
    from gpu_util import TORCH_DT, say, to_f64, upload
    say(f"pool beyond 4 GiB {dt} G={Hq // Hkv} D={D} bs={bs}")
    L = [1, 40, 333, 1000]
    c = make_case(B=4, Hq=Hq, Hkv=Hkv, D=D, bs=bs, dtype=dt, context_lens=L, softcap=cap,
                  partition_size=P, seed=41, new_rows=True)
    page = bs * Hkv * D * 2
    NB_big = (9 << 29) // page + 7           # 4.5 GiB per cache, plus a few pages
    assert NB_big * page > (1 << 32)
    dev = torch.device("cuda")
    tdt = TORCH_DT[dt]
    kc = torch.full((NB_big, bs, Hkv, D), float("nan"), dtype=tdt, device=dev)
    vc = torch.full((NB_big, bs, Hkv, D), float("nan"), dtype=tdt, device=dev)
    # the case's pool block i -> block NB_big - 1 - i (the top of the pool)
    remap = NB_big - 1 - np.arange(c.NB)
    ids = torch.from_numpy(remap).to(dev)
    kc[ids] = upload(c.k_cache, dt)
    vc[ids] = upload(c.v_cache, dt)
    bt = torch.from_numpy(np.where(c.block_tables >= 0,
                                   remap[np.maximum(c.block_tables, 0)], -1).astype(np.int32)).to(dev)
    slots = np.where(c.slot_mapping >= 0,
                     remap[c.slot_mapping // bs] * bs + c.slot_mapping % bs, -1).astype(np.int64)
    assert slots.max() * Hkv * D * 2 > (1 << 32)
    pa.reshape_and_cache(upload(c.key, dt), upload(c.value, dt), kc, vc,
                         torch.from_numpy(slots).to(dev))
    out = pa.decode(upload(c.q, dt), kc, vc, bt, torch.from_numpy(c.context_lens).to(dev),
                    c.scale, c.softcap, c.window, partition_size=P,
                    max_context_len=c.max_context_len)
    torch.cuda.synchronize()
    check(c, to_f64(out))
    # copy-on-write between two blocks above 4 GiB: bit-exact
    src, dst = int(remap[0]), int(NB_big - 1 - c.NB - 3)
    pa.copy_blocks(kc, vc, torch.tensor([[src, dst]], dtype=torch.int64, device=dev))
    torch.cuda.synchronize()
    assert torch.equal(kc[dst].view(torch.int16), kc[src].view(torch.int16))
    assert torch.equal(vc[dst].view(torch.int16), vc[src].view(torch.int16))
    del kc, vc
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dt,Hq,Hkv,D,P", [("bf16", 8, 2, 128, 0), ("f32", 4, 4, 64, 512),
                                           ("f16", 16, 2, 64, 256)])
def test_block_size_256(dt, Hq, Hkv, D, P):
    """The largest supported block size: chunks inside one page, contexts of
    one page, a ragged page tail and several pages."""
    from gpu_util import say
    say(f"block size 256 {dt} G={Hq // Hkv} D={D} P={P}")
    L = [1, 255, 256, 257, 700, 1300]
    c = make_case(B=len(L), Hq=Hq, Hkv=Hkv, D=D, bs=256, dtype=dt, context_lens=L,
                  softcap=30.0, partition_size=P, seed=43, new_rows=True, extra_table_cols=1)
    check(c, gpu(c))
