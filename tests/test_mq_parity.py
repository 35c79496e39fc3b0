"""Multi-query paged attention on the GPU (pa_mq_attention) against the
oracle: each new token attends causally to the keys up to its own position.

Both paths are covered: the tiled matrix-core path (f16/bf16, pages of 16+
tokens, any group size) and the per-token path (every other shape, or
PA_MQ_TILED=0).  New tokens' K/V rows land through pa_reshape_and_cache
first, into slots the generator poisoned."""
import os

import numpy as np
import pytest

import oracle
from oracle import oracle as O
from workloads import make_mq_case, mq_workload

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "f16": 2e-2, "bf16": 2e-2}


class DeviceMQ:
    def __init__(self, c):
        import torch
        from gpu_util import upload
        self.c = c
        self.q = upload(c.q, c.dtype)
        self.k_cache = upload(c.k_cache, c.dtype)
        self.v_cache = upload(c.v_cache, c.dtype)
        self.block_tables = torch.from_numpy(c.block_tables).cuda()
        self.context_lens = torch.from_numpy(c.context_lens).cuda()
        self.query_start = torch.from_numpy(c.query_start).cuda()
        self.key = self.value = self.slots = None
        if c.slot_mapping is not None:
            self.key = upload(c.key, c.dtype)
            self.value = upload(c.value, c.dtype)
            self.slots = torch.from_numpy(c.slot_mapping).cuda()

    def run(self, partition_size=None, tiled=None, out=None, max_query_len=None, shared=None,
            env=None):
        """tiled: matrix-core path (True) or per token (False); shared: force
        the workgroup-shared (True) or per-wavefront (False) tiled kernel;
        env: further switches for this call."""
        import torch
        import paged_kv_decode_pa_amd as pa
        c = self.c
        env = dict(env or {})
        if tiled is not None:
            env["PA_MQ_TILED"] = "1" if tiled else "0"
        if shared is not None:
            env["PA_MQ_WG"] = "1" if shared else "0"
        os.environ.update(env)
        try:
            if self.slots is not None:
                pa.reshape_and_cache(self.key, self.value, self.k_cache, self.v_cache, self.slots)
            P = c.partition_size if partition_size is None else partition_size
            out = pa.mq_attention(self.q, self.query_start, self.k_cache, self.v_cache,
                                  self.block_tables, self.context_lens, c.scale, c.softcap,
                                  c.window, partition_size=P, max_context_len=c.max_context_len,
                                  max_query_len=max_query_len or max(1, c.max_query_len), out=out)
            torch.cuda.synchronize()
        finally:
            for k in env:
                os.environ.pop(k, None)
        return out


def check(got_t, want, dtype, rows=None):
    from gpu_util import to_f64
    got = to_f64(got_t)
    # every output row, compared or not, must be finite: a read of a
    # NaN-poisoned slot anywhere shows up here
    assert np.isfinite(got).all(), "non-finite output"
    if rows is not None:
        got = got[rows]
    err = np.abs(got - want).max() if got.size else 0.0
    assert err <= TOL[dtype], f"max abs error {err:.3g} > {TOL[dtype]}"
    return err


# (dtype, G, D, bs, softcap, window, partition, context lens, query lens)
SHAPES = [
    ("bf16", 2, 256, 16, 50.0, 0, 0, [40, 77, 5, 130], [5, 77, 1, 9]),
    ("bf16", 2, 256, 16, 50.0, 0, 32, [40, 77, 5, 130], [5, 77, 1, 9]),
    ("f16", 8, 64, 32, 0.0, 0, 0, [300, 64, 33], [17, 64, 2]),
    ("f16", 8, 64, 32, 0.0, 0, 64, [300, 64, 33], [17, 64, 2]),
    ("bf16", 4, 128, 32, 30.0, 45, 0, [200, 97, 160], [33, 97, 6]),
    ("bf16", 4, 128, 16, 0.0, 20, 48, [200, 97, 160], [33, 50, 6]),
    ("f16", 1, 128, 64, 0.0, 0, 128, [250, 129], [70, 129]),
    ("bf16", 16, 64, 16, 20.0, 0, 0, [90, 31, 46], [3, 31, 5]),
    ("bf16", 3, 64, 16, 0.0, 0, 32, [70, 48], [11, 48]),     # group of 3 heads
    ("f16", 2, 64, 16, 0.0, 7, 16, [61, 18, 9], [13, 18, 9]),
    # head_dim 64 over 32-token pages: 64-key chunks spanning two pages on
    # the shared kernel, with windows and partitions that start mid-chunk
    ("f16", 4, 64, 32, 0.0, 40, 96, [300, 97, 64], [70, 97, 5]),
    ("bf16", 8, 64, 32, 30.0, 0, 96, [333, 150, 40], [150, 150, 7]),
]


def _id(s):
    return f"{s[0]}-g{s[1]}-d{s[2]}-bs{s[3]}-c{int(s[4])}-w{s[5]}-p{s[6]}"


# path -> (tiled, shared, extra switches): the per-wavefront kernel runs with
# one wavefront per KV head by default ("wave") or split chunks ("wave-split")
PATHS = {"shared": (True, True, None), "wave": (True, False, None),
         "wave-split": (True, False, {"PA_MQ_HEADS": "0"}), "auto": (True, None, None),
         "pertoken": (False, None, None)}


@pytest.mark.parametrize("shape", SHAPES, ids=[_id(s) for s in SHAPES])
@pytest.mark.parametrize("path", list(PATHS))
def test_mq_shapes(shape, path):
    from gpu_util import say
    dtype, G, D, bs, cap, W, P, L, n = shape
    tiled, shared, env = PATHS[path]
    if not tiled and G not in (1, 2, 4, 8, 16):
        pytest.skip("the per-token path takes the decode group sizes")
    say(f"mq {_id(shape)} path={path}")
    Hkv = 2
    c = make_mq_case(Hq=G * Hkv, Hkv=Hkv, D=D, bs=bs, dtype=dtype, context_lens=L, query_lens=n,
                     softcap=cap, window=W, partition_size=P, seed=D + G + bs + W,
                     new_rows=True)
    got = DeviceMQ(c).run(tiled=tiled, shared=shared, env=env)
    check(got, oracle.multi_query_case(c), dtype)


@pytest.mark.parametrize("dtype,bs", [("f32", 16), ("f32", 1), ("bf16", 8), ("f16", 1)])
def test_mq_per_token_only_shapes(dtype, bs):
    """f32 and pages under 16 tokens always run per token."""
    from gpu_util import say
    say(f"mq per-token {dtype} bs={bs}")
    c = make_mq_case(Hq=8, Hkv=2, D=64, bs=bs, dtype=dtype, context_lens=[45, 100, 17],
                     query_lens=[9, 100, 3], softcap=10.0, partition_size=32 if bs <= 32 else 0,
                     seed=5 + bs, new_rows=True)
    got = DeviceMQ(c).run()
    check(got, oracle.multi_query_case(c), dtype)


def test_mq_one_token_matches_decode_bitwise():
    """With one new token per sequence the per-token path runs the decode
    kernels on the same units: bit-identical to pa_decode."""
    import torch
    import paged_kv_decode_pa_amd as pa
    from gpu_util import say
    say("mq one token vs decode")
    L = [33, 500, 1, 257, 64]
    c = make_mq_case(Hq=8, Hkv=4, D=256, bs=16, dtype="bf16", context_lens=L,
                     query_lens=[1] * len(L), softcap=50.0, partition_size=128, seed=9)
    d = DeviceMQ(c)
    got = d.run()
    dec = pa.decode(d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, c.scale,
                    c.softcap, c.window, partition_size=128, max_context_len=c.max_context_len)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), dec.view(torch.int16))


def test_mq_empty_sequences_and_no_tokens():
    import torch
    import paged_kv_decode_pa_amd as pa
    from gpu_util import say
    say("mq empty sequences")
    c = make_mq_case(Hq=4, Hkv=2, D=64, bs=16, dtype="bf16", context_lens=[20, 0, 35, 9],
                     query_lens=[4, 0, 0, 9], partition_size=16, seed=2, new_rows=True)
    for tiled, shared in ((True, True), (True, False), (False, None)):
        check(DeviceMQ(c).run(tiled=tiled, shared=shared), oracle.multi_query_case(c), "bf16")
    z = make_mq_case(Hq=4, Hkv=2, D=64, bs=16, dtype="bf16", context_lens=[20, 7],
                     query_lens=[0, 0], seed=3)
    out = DeviceMQ(z).run()
    assert out.shape == (0, 4, 64)


def test_mq_chunked_prefill_matches_whole_prompt():
    """A 300-token prompt prefilled in chunks of 128 (each chunk attending to
    the cache so far plus itself) gives the rows of one whole-prompt
    prefill."""
    import torch
    import paged_kv_decode_pa_amd as pa
    from gpu_util import say, to_f64, upload
    say("mq chunked prefill")
    Lp = 300
    whole = make_mq_case(Hq=8, Hkv=4, D=128, bs=32, dtype="f16", context_lens=[Lp],
                         query_lens=[Lp], seed=11, new_rows=True)
    ref = to_f64(DeviceMQ(whole).run())
    d = DeviceMQ(whole)
    pa.reshape_and_cache(d.key, d.value, d.k_cache, d.v_cache, d.slots)
    rows = []
    for a in range(0, Lp, 128):
        e = min(Lp, a + 128)
        qs = torch.tensor([0, e - a], dtype=torch.int32, device="cuda")
        cl = torch.tensor([e], dtype=torch.int32, device="cuda")
        o = pa.mq_attention(d.q[a:e].contiguous(), qs, d.k_cache, d.v_cache, d.block_tables, cl,
                            whole.scale, 0.0, 0, partition_size=64, max_context_len=e,
                            max_query_len=e - a)
        rows.append(to_f64(o))
    got = np.concatenate(rows)
    assert np.abs(got - ref).max() <= 2e-2
    np.testing.assert_allclose(ref, oracle.multi_query_case(whole), rtol=0, atol=2e-2)


def test_mq_output_guard_band_untouched():
    import torch
    from gpu_util import say
    say("mq guard band")
    c = make_mq_case(Hq=8, Hkv=2, D=128, bs=16, dtype="bf16", context_lens=[50, 70],
                     query_lens=[7, 30], partition_size=32, seed=4, new_rows=True)
    d = DeviceMQ(c)
    big = torch.full((c.T + 3, 8, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    d.run(out=big[:c.T])
    assert torch.all(big[c.T:] == 7.0)
    check(big[:c.T], oracle.multi_query_case(c), "bf16")


def _sampled(c, k, seed):
    """Oracle rows for k sampled tokens (each computed on its own)."""
    kc, vc = O.reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping)
    rng = np.random.default_rng(seed)
    toks = np.sort(rng.choice(c.T, size=min(k, c.T), replace=False))
    # always the first and last token of the longest sequence
    b = int(np.argmax(c.query_lens))
    toks = np.unique(np.concatenate([toks, [c.query_start[b], c.query_start[b + 1] - 1]]))
    want = []
    for t in toks:
        b = int(np.searchsorted(c.query_start, t, side="right") - 1)
        pos = int(c.context_lens[b]) - int(c.query_lens[b]) + int(t - c.query_start[b])
        want.append(O.attend(c.q[t], kc, vc, c.block_tables, b, pos + 1, c.scale, c.softcap,
                             c.window, c.dtype))
    return toks, np.stack(want)


@pytest.mark.parametrize("name", ["spec5", "chunk512"])
def test_mq_workloads_every_token(name):
    """The speculative-verification (2,560 tokens) and chunked-prefill (575
    tokens) workloads at full size, launched as the bench launches them:
    every token against the oracle."""
    from gpu_util import say
    say(f"mq workload {name}")
    c = mq_workload(name)
    got = DeviceMQ(c).run()
    check(got, oracle.multi_query_case(c), c.dtype)


def test_mq_workload_prefill():
    """Whole-prompt prefill, 4 x 2,048 tokens: every token of the first
    prompt against the oracle, 48 sampled tokens of the others, and every
    output row finite."""
    from gpu_util import say
    say("mq workload prefill")
    c = mq_workload("prefill")
    got = DeviceMQ(c).run()
    kc, vc = O.reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping)
    n0 = int(c.query_start[1])
    want0 = O.multi_query(c.q[:n0], c.query_start[:2], kc, vc, c.block_tables[:1],
                          c.context_lens[:1], c.scale, c.softcap, c.window, c.dtype)
    check(got, want0, c.dtype, rows=np.arange(n0))
    toks, want = _sampled(c, 48, 7)
    check(got, want, c.dtype, rows=toks)


def test_mq_many_sequences():
    """More sequences than the plan stages in LDS (4,096) and than one plan
    slice (1,024): every token still finds its sequence."""
    from gpu_util import say
    say("mq many sequences")
    rng = np.random.default_rng(77)
    B = 4500
    L = rng.integers(1, 40, size=B)
    n = np.minimum(L, rng.integers(0, 4, size=B))
    c = make_mq_case(Hq=4, Hkv=2, D=64, bs=16, dtype="bf16", context_lens=L, query_lens=n,
                     partition_size=0, seed=78, new_rows=True, poison=False)
    for tiled, shared in ((True, False), (False, None)):
        got = DeviceMQ(c).run(tiled=tiled, shared=shared)
        toks, want = _sampled(c, 200, 5)
        check(got, want, "bf16", rows=toks)


@pytest.mark.parametrize("P,W", [(0, 0), (64, 0), (64, 100), (512, 0)])
def test_mq_mixed_batch(P, W):
    """Prompt chunks beside decoding sequences, empty sequences and drafts of
    a few tokens in one call, on the shared kernel and on the per-token
    path: every token matches the oracle."""
    from gpu_util import say
    say(f"mq mixed batch P={P} W={W}")
    rng = np.random.default_rng(300 + P + W)
    L = [700, 1, 300, 64, 0, 1200, 33, 500, 90, 257]
    n = [96, 1, 1, 64, 0, 1, 5, 1, 40, 1]
    c = make_mq_case(Hq=8, Hkv=4, D=256, bs=16, dtype="bf16", context_lens=L, query_lens=n,
                     softcap=50.0, window=W, partition_size=P, seed=int(rng.integers(1 << 30)),
                     new_rows=True)
    want = oracle.multi_query_case(c)
    check(DeviceMQ(c).run(shared=True), want, "bf16")
    check(DeviceMQ(c).run(tiled=False), want, "bf16")


@pytest.mark.parametrize("P,W", [(64, 0), (64, 100), (48, 20)])
def test_mq_unit_list_matches_plan_order(P, W):
    """With keys split, the shared kernel walks the plan's sorted (tile,
    partition) list; each unit's results do not depend on when it runs, so
    the output equals, bit for bit, that of the grid in plan order with
    partitions slowest (PA_MQ_UNITS=0), and matches the oracle."""
    from gpu_util import say, to_f64
    say(f"mq unit list P={P} W={W}")
    rng = np.random.default_rng(900 + P + W)
    L = [700, 1, 300, 64, 0, 1200, 33, 500, 90, 257]
    n = [96, 1, 1, 64, 0, 1, 5, 1, 40, 1]
    c = make_mq_case(Hq=8, Hkv=4, D=256, bs=16, dtype="bf16", context_lens=L, query_lens=n,
                     softcap=50.0, window=W, partition_size=P, seed=int(rng.integers(1 << 30)),
                     new_rows=True)
    dev = DeviceMQ(c)
    by_units = to_f64(dev.run(shared=True))
    in_order = to_f64(dev.run(shared=True, env={"PA_MQ_UNITS": "0"}))
    assert np.array_equal(by_units, in_order)
    check(dev.run(shared=True), oracle.multi_query_case(c), "bf16")


def _bits(t):
    import torch
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


@pytest.mark.parametrize("P,W,tiled", [(64, 100, True), (0, 0, True), (32, 0, False)])
def test_mq_step_matches_reshape_then_attention(P, W, tiled):
    """pa_mq_step, whose plan launch also writes the new K/V rows, leaves the
    caches and the output bit for bit as reshape_and_cache followed by
    pa_mq_attention do; two extra rows with slot -1 and a slot past the pool
    are skipped by both.  The output also matches the oracle."""
    import torch
    import paged_kv_decode_pa_amd as pa
    from gpu_util import say
    say(f"mq step P={P} W={W} tiled={tiled}")
    rng = np.random.default_rng(1200 + P + W)
    L = [700, 1, 300, 64, 0, 1200, 33, 500, 90, 257]
    n = [96, 1, 1, 64, 0, 1, 5, 1, 40, 1]
    dt = "bf16" if tiled else "f16"
    c = make_mq_case(Hq=8, Hkv=4, D=128, bs=16, dtype=dt, context_lens=L, query_lens=n,
                     softcap=30.0, window=W, partition_size=P, seed=int(rng.integers(1 << 30)),
                     new_rows=True)
    dev = DeviceMQ(c)
    NB, bs = c.k_cache.shape[:2]
    key = torch.cat([dev.key, dev.key[:2]])
    value = torch.cat([dev.value, dev.value[:2]])
    slots = torch.cat([dev.slots, torch.tensor([-1, NB * bs + 3], dtype=torch.int64,
                                               device=dev.slots.device)])
    kc0, vc0 = dev.k_cache.clone(), dev.v_cache.clone()
    args = (dev.q, dev.query_start, dev.k_cache, dev.v_cache, dev.block_tables,
            dev.context_lens, c.scale, c.softcap, c.window)
    kw = dict(partition_size=P, max_context_len=c.max_context_len,
              max_query_len=max(1, c.max_query_len))
    os.environ["PA_MQ_TILED"] = "1" if tiled else "0"
    try:
        pa.reshape_and_cache(key, value, dev.k_cache, dev.v_cache, slots)
        out_a = pa.mq_attention(*args, **kw)
        torch.cuda.synchronize()
        kc_a, vc_a = dev.k_cache.clone(), dev.v_cache.clone()
        dev.k_cache.copy_(kc0)
        dev.v_cache.copy_(vc0)
        out_b = pa.mq_attention(*args, key=key, value=value, slot_mapping=slots, **kw)
        torch.cuda.synchronize()
        assert torch.equal(_bits(dev.k_cache), _bits(kc_a))
        assert torch.equal(_bits(dev.v_cache), _bits(vc_a))
        # the prebuilt step object, run twice on the original caches
        dev.k_cache.copy_(kc0)
        dev.v_cache.copy_(vc0)
        st = pa.MQStep(*args, key=key, value=value, slot_mapping=slots, **kw)
        st.run()
        out_c = st.run().clone()
        torch.cuda.synchronize()
    finally:
        os.environ.pop("PA_MQ_TILED", None)
    assert torch.equal(_bits(dev.k_cache), _bits(kc_a))
    assert torch.equal(_bits(dev.v_cache), _bits(vc_a))
    assert torch.equal(_bits(out_b), _bits(out_a))
    assert torch.equal(_bits(out_c), _bits(out_a))
    check(out_b, oracle.multi_query_case(c), dt)


@pytest.mark.parametrize("B", [400, 700])
@pytest.mark.parametrize("path", ["wave", "wave-split"])
def test_mq_resident_order(B, path):
    """Per-wavefront kernel, grids of several resident rounds (one tile per
    sequence, about 0.8 B tiles; a round is 256 workgroups):
    the position -> tile map that reverses odd rounds (a partial one
    included) covers every tile once.  Output matches the oracle, and
    equals the plan-order launch (PA_MQ_RESIDENT=0) bit for bit."""
    from gpu_util import say, to_f64
    say(f"mq resident order B={B} path={path}")
    rng = np.random.default_rng(900 + B)
    n = rng.integers(0, 5, size=B)
    L = n + rng.integers(0, 120, size=B)
    c = make_mq_case(Hq=4, Hkv=2, D=64, bs=16, dtype="bf16", context_lens=L, query_lens=n,
                     softcap=30.0, partition_size=0, seed=int(rng.integers(1 << 30)),
                     new_rows=True)
    tiled, shared, env = PATHS[path]
    dev = DeviceMQ(c)
    got = dev.run(tiled=tiled, shared=shared, env=env)
    check(got, oracle.multi_query_case(c), "bf16")
    ref = dev.run(tiled=tiled, shared=shared, env={**(env or {}), "PA_MQ_RESIDENT": "0"})
    assert np.array_equal(to_f64(got), to_f64(ref))


@pytest.mark.parametrize("cap", [0.0, 30.0])
def test_mq_shared_kernel_wide_logits(cap):
    """Logits 16x the usual spread (scale 2 at head_dim 64): a row's running
    maximum then jumps by more than the kernel's slack within a prompt, so
    both the rescale and the keep-the-reference branches of the shared
    kernel's online softmax run, with and without soft-capping."""
    from gpu_util import say
    say(f"mq shared kernel wide logits cap={cap}")
    c = make_mq_case(Hq=16, Hkv=2, D=64, bs=32, dtype="f16", context_lens=[300, 170],
                     query_lens=[300, 90], scale=2.0, softcap=cap, partition_size=128,
                     seed=4242 + int(cap), new_rows=True)
    want = oracle.multi_query_case(c)
    check(DeviceMQ(c).run(shared=True), want, "f16")
    check(DeviceMQ(c).run(shared=True, partition_size=0), oracle.multi_query_case(c), "f16")
