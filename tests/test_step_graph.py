"""The layer step (reshape_and_cache + decode + merge) through pa_step and
through a captured HIP graph: every replay equals an eager pa_step on the
same inputs bit for bit, with other eager work and synchronisations between
replays, and replays follow input changes (nothing is cached)."""
import numpy as np
import pytest

import oracle
from workloads import encode, make_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("P", [0, 128])
def test_step_graph_replays_match_eager(P):
    import torch
    import paged_kv_decode_pa_amd as pa
    from gpu_util import DeviceCase, say, to_f64, upload
    say(f"step graph P={P}")
    c = make_case(B=12, Hq=8, Hkv=4, D=256, bs=16, dtype="bf16",
                  context_lens=[5, 900, 130, 17, 640, 1, 333, 700, 256, 257, 48, 999],
                  softcap=50.0, partition_size=P, seed=31, new_rows=True)
    dc = DeviceCase(c)
    step = pa.Step(dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, c.scale,
                   c.softcap, c.window, partition_size=P, max_context_len=c.max_context_len,
                   key=dc.key, value=dc.value, slot_mapping=dc.slot_mapping)
    # eager pa_step on the same buffers (its own output): the reference the
    # replays must equal bit for bit
    eager_step = pa.Step(dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                         c.scale, c.softcap, c.window, partition_size=P,
                         max_context_len=c.max_context_len, key=dc.key, value=dc.value,
                         slot_mapping=dc.slot_mapping)
    s = torch.cuda.Stream()
    step.capture(s)
    rng = np.random.default_rng(5)
    for r in range(4):
        # new query contents (same buffer), then eager reference and replay
        newq = encode(rng.standard_normal(c.q.shape).astype(np.float32), "bf16")
        dc.q.copy_(upload(newq, "bf16"))
        c.q = newq
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            got = to_f64(step.replay(s).clone())
        s.synchronize()
        eager = to_f64(eager_step.run().clone())
        torch.cuda.synchronize()
        assert np.array_equal(got, eager), f"replay {r} differs from eager"
        want = oracle.decode_case(c)
        assert np.abs(got - want).max() <= 2e-2
        # and so do the separate entry points
        sep = to_f64(pa.decode(dc.q, dc.k_cache, dc.v_cache, dc.block_tables,
                               dc.context_lens, c.scale, c.softcap, c.window,
                               partition_size=P, max_context_len=c.max_context_len))
        assert np.array_equal(got, sep), f"replay {r} differs from pa_decode + reduce"
        # unrelated eager work between replays
        x = torch.randn(1 << 20, device="cuda")
        (x * 2).sum().item()
    step.close()


def test_step_runs_eagerly():
    import torch
    import paged_kv_decode_pa_amd as pa
    from gpu_util import DeviceCase, say, to_f64
    say("step eager")
    c = make_case(B=5, Hq=32, Hkv=4, D=64, bs=32, dtype="f16",
                  context_lens=[3000, 40, 1, 777, 2048], partition_size=512, seed=32,
                  new_rows=True)
    dc = DeviceCase(c)
    step = pa.Step(dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, c.scale,
                   c.softcap, c.window, partition_size=512, max_context_len=c.max_context_len,
                   key=dc.key, value=dc.value, slot_mapping=dc.slot_mapping)
    got = to_f64(step.run())
    torch.cuda.synchronize()
    assert np.abs(got - oracle.decode_case(c)).max() <= 2e-2


def test_graph_of_several_layer_steps():
    """Three layer steps with their own buffers and shapes (two decode
    layers of different widths and a long-context one with split keys)
    captured into one graph: every replay equals each step run eagerly, bit
    for bit, with new queries and unrelated eager work between replays."""
    import torch
    import paged_kv_decode_pa_amd as pa
    from gpu_util import DeviceCase, say, to_f64, upload
    say("graph of three layer steps")
    cases = [
        make_case(B=7, Hq=8, Hkv=4, D=256, bs=16, dtype="bf16",
                  context_lens=[5, 900, 130, 17, 640, 1, 333], softcap=50.0, partition_size=0,
                  seed=41, new_rows=True),
        make_case(B=4, Hq=8, Hkv=2, D=128, bs=16, dtype="f16", context_lens=[77, 3, 260, 1000],
                  partition_size=128, seed=42, new_rows=True),
        make_case(B=3, Hq=32, Hkv=4, D=64, bs=32, dtype="f16", context_lens=[4000, 70, 1500],
                  partition_size=512, seed=43, new_rows=True),
    ]
    devs = [DeviceCase(c) for c in cases]

    def mk(c, dc):
        return pa.Step(dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, c.scale,
                       c.softcap, c.window, partition_size=c.partition_size,
                       max_context_len=c.max_context_len, key=dc.key, value=dc.value,
                       slot_mapping=dc.slot_mapping)
    steps = [mk(c, dc) for c, dc in zip(cases, devs)]
    eager = [mk(c, dc) for c, dc in zip(cases, devs)]
    s = torch.cuda.Stream()
    g = pa.StepGraph(steps, s)
    rng = np.random.default_rng(6)
    for r in range(3):
        for c, dc in zip(cases, devs):
            newq = encode(rng.standard_normal(c.q.shape).astype(np.float32), c.dtype)
            dc.q.copy_(upload(newq, c.dtype))
            c.q = newq
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay(s)
        s.synchronize()
        for i, (c, st, ref) in enumerate(zip(cases, steps, eager)):
            got = to_f64(st.out.clone())
            want_bits = to_f64(ref.run().clone())
            torch.cuda.synchronize()
            assert np.array_equal(got, want_bits), f"replay {r}, step {i} differs from eager"
            assert np.abs(got - oracle.decode_case(c)).max() <= 2e-2
        x = torch.randn(1 << 20, device="cuda")
        (x * 2).sum().item()
    g.close()
