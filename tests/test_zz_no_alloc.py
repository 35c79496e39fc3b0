"""pa_step_static (the layer step with its scratch in the library's static
per-GPU array, for callers that cannot allocate) against pa_step with a
caller workspace: identical bits, and the oracle's tolerance, on two calls in
a row -- the second with a smaller input, so it runs over what the first
left in the array."""
import numpy as np
import pytest

import oracle
from workloads import make_case

pytestmark = pytest.mark.gpu


def _step(c):
    import paged_kv_decode_pa_amd as pa
    from gpu_util import DeviceCase
    dc = DeviceCase(c)
    return pa.Step(dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, c.scale,
                   c.softcap, c.window, partition_size=c.partition_size,
                   max_context_len=c.max_context_len, key=dc.key, value=dc.value,
                   slot_mapping=dc.slot_mapping)


def _both(c):
    """Run the case through pa_step (own workspace) and through
    pa_step_static, each on freshly uploaded buffers."""
    import torch
    from gpu_util import to_f64
    ref = _step(c)
    ref.run()
    st = _step(c)
    st.run_static()
    torch.cuda.synchronize()
    return to_f64(ref.out), to_f64(st.out), ref.out, st.out


@pytest.mark.parametrize("P", [0, 64])
def test_static_step_equals_workspace_step_twice(P):
    import torch
    from gpu_util import say
    first = make_case(B=40, Hq=8, Hkv=4, D=256, bs=16, dtype="bf16",
                      context_lens=list(range(1, 1001, 25)), softcap=50.0, scale=1 / 16,
                      seed=7001 + P, new_rows=True, partition_size=P)
    second = make_case(B=5, Hq=8, Hkv=4, D=256, bs=16, dtype="bf16",
                       context_lens=[1, 9, 130, 70, 300], softcap=50.0, scale=1 / 16,
                       seed=7002 + P, new_rows=True, partition_size=P)
    for name, c in (("first", first), ("second, smaller", second)):
        say(f"pa_step_static {name} call: B={c.B} P={P}")
        a, b, ta, tb = _both(c)
        assert torch.equal(ta.view(torch.int16), tb.view(torch.int16)), "bits differ from pa_step"
        want = oracle.decode_case(c)
        assert np.isfinite(b).all()
        assert np.abs(b - want).max() <= 2e-2


def test_static_step_long_context_partials():
    """The matrix-core decode over split keys (partials in the array), then a
    smaller float32 case on the vector kernel."""
    import torch
    from gpu_util import say
    big = make_case(B=6, Hq=32, Hkv=4, D=64, bs=32, dtype="f16",
                    context_lens=[9000, 40, 4097, 1, 12000, 600], scale=1 / 8,
                    seed=7003, new_rows=True, partition_size=512)
    small = make_case(B=3, Hq=8, Hkv=2, D=64, bs=16, dtype="f32", context_lens=[17, 255, 64],
                      scale=1 / 8, seed=7004, new_rows=True, partition_size=32)
    for c, tol in ((big, 2e-2), (small, 1e-4)):
        say(f"pa_step_static {c.dtype} B={c.B} P={c.partition_size}")
        a, b, ta, tb = _both(c)
        assert np.array_equal(a, b), "differs from pa_step"
        assert np.isfinite(b).all()
        assert np.abs(b - oracle.decode_case(c)).max() <= tol


def test_static_step_rejects_oversize():
    """A step whose scratch exceeds the array is refused before anything
    runs (PA_ESCRATCH), and the output is left untouched."""
    import torch
    import paged_kv_decode_pa_amd as pa
    from paged_kv_decode_pa_amd import _lib
    from gpu_util import say
    say("pa_step_static oversize")
    c = make_case(B=4, Hq=8, Hkv=4, D=256, bs=16, dtype="bf16", context_lens=[1, 2, 3, 4],
                  seed=7005, partition_size=16)
    st = _step(c)
    st.out.fill_(3.0)
    st.args.max_context_len = 1 << 20       # host-side bound only: sizes the scratch
    st.args.max_blocks_per_seq = 1 << 16
    st.args.num_seqs = 4
    need = pa.workspace_size(c.B, c.Hq, c.D, 1 << 20, 16)
    assert need > _lib.PA_STATIC_SCRATCH_BYTES
    with pytest.raises(pa.PaError) as e:
        st.run_static()
    assert e.value.status == -5
    torch.cuda.synchronize()
    assert torch.all(st.out == 3.0)
