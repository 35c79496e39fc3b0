"""reshape_and_cache on the GPU against the oracle's scatter: bit-exact over
the whole pool (untouched slots unchanged, -1 rows skipped, NaN payloads
kept)."""
import numpy as np
import pytest

import oracle
from workloads import encode, make_case, workload

pytestmark = pytest.mark.gpu


def _run(key, value, kc, vc, slots, dtype):
    import torch
    import paged_kv_decode_pa_amd as pa
    from gpu_util import upload
    dk, dv = upload(kc, dtype), upload(vc, dtype)
    pa.reshape_and_cache(upload(key, dtype), upload(value, dtype), dk, dv,
                         torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    back = lambda t: (t.view(torch.int16).cpu().numpy().view(np.uint16)
                      if dtype != "f32" else t.cpu().numpy())
    return back(dk), back(dv)


@pytest.mark.parametrize("dtype,D,bs,Hkv", [("f32", 64, 16, 2), ("f16", 128, 1, 4),
                                             ("bf16", 256, 16, 4), ("bf16", 64, 32, 8)])
def test_reshape_bit_exact(dtype, D, bs, Hkv):
    from gpu_util import say
    say(f"reshape {dtype} D={D} bs={bs} Hkv={Hkv}")
    rng = np.random.default_rng(D + bs)
    NB, T = 37, 50
    kc = encode(rng.standard_normal((NB, bs, Hkv, D)).astype(np.float32), dtype)
    vc = encode(rng.standard_normal((NB, bs, Hkv, D)).astype(np.float32), dtype)
    key = encode(rng.standard_normal((T, Hkv, D)).astype(np.float32), dtype)
    value = encode(rng.standard_normal((T, Hkv, D)).astype(np.float32), dtype)
    if dtype == "f32":
        key[3, 0, 5] = np.frombuffer(np.uint32(0x7FA00001).tobytes(), np.float32)[0]
    else:
        key[3, 0, 5] = np.uint16(0x7D01)  # NaN payload must survive
    T_ = min(T, NB * bs)
    slots = rng.choice(NB * bs, size=T_, replace=False).astype(np.int64)
    slots[::7] = -1
    key, value = key[:T_], value[:T_]
    gk, gv = _run(key, value, kc, vc, slots, dtype)
    wk, wv = oracle.reshape_and_cache(key, value, kc, vc, slots)
    assert gk.tobytes() == wk.tobytes()
    assert gv.tobytes() == wv.tobytes()


def test_reshape_gemma_global_new_rows():
    """The 64 new rows of the Gemma-2-2B global-layer workload (bf16)."""
    from gpu_util import say
    say("reshape workload 2")
    c = workload(2)
    gk, gv = _run(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping, "bf16")
    wk, wv = oracle.reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping)
    assert gk.tobytes() == wk.tobytes()
    assert gv.tobytes() == wv.tobytes()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_reshape_skips_slots_outside_the_pool(dtype):
    """Slots past the pool's end (num_blocks * block_size and beyond) and
    negative slots other than -1 are skipped, as -1 is: the caches equal the
    oracle's scatter bit for bit.  The kernel tests the slot against the
    pool size before it forms an address, so these are in-bounds skips."""
    from gpu_util import say
    say(f"reshape out-of-pool slots {dtype}")
    rng = np.random.default_rng(404)
    NB, bs, Hkv, D = 11, 16, 2, 64
    kc = encode(rng.standard_normal((NB, bs, Hkv, D)).astype(np.float32), dtype)
    vc = encode(rng.standard_normal((NB, bs, Hkv, D)).astype(np.float32), dtype)
    slots = np.array([NB * bs, 5, -1, NB * bs + 1, -7, NB * bs - 1, 1 << 40, 0, (1 << 62)],
                     dtype=np.int64)
    T = len(slots)
    key = encode(rng.standard_normal((T, Hkv, D)).astype(np.float32), dtype)
    value = encode(rng.standard_normal((T, Hkv, D)).astype(np.float32), dtype)
    gk, gv = _run(key, value, kc, vc, slots, dtype)
    wk, wv = oracle.reshape_and_cache(key, value, kc, vc, slots)
    assert gk.tobytes() == wk.tobytes()
    assert gv.tobytes() == wv.tobytes()


def test_step_new_rows_skip_slots_outside_the_pool():
    """The layer step's preparation launch writes new rows with the same
    rule: a case whose new-row slots include out-of-pool values decodes like
    the oracle's step (those rows never land; the sequences whose slot was
    replaced read the poisoned slot, so only the others are compared) and
    leaves the caches equal to the oracle's scatter."""
    import torch
    import paged_kv_decode_pa_amd as pa
    from gpu_util import DeviceCase, say, to_f64
    say("pa_step out-of-pool slots")
    c = make_case(B=6, Hq=8, Hkv=4, D=256, bs=16, dtype="bf16",
                  context_lens=[3, 40, 100, 17, 64, 200], softcap=50.0, scale=1 / 16,
                  seed=4040, new_rows=True, partition_size=0)
    bad = [1, 4]
    c.slot_mapping = c.slot_mapping.copy()
    c.slot_mapping[bad[0]] = c.NB * c.bs
    c.slot_mapping[bad[1]] = c.NB * c.bs + 12345
    dc = DeviceCase(c)
    step = pa.Step(dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens, c.scale,
                   c.softcap, c.window, partition_size=0, max_context_len=c.max_context_len,
                   key=dc.key, value=dc.value, slot_mapping=dc.slot_mapping)
    step.run()
    torch.cuda.synchronize()
    got = to_f64(step.out)
    keep = [b for b in range(c.B) if b not in bad]
    want = oracle.decode_case(c, seqs=keep)
    assert np.isfinite(got[keep]).all()
    assert np.abs(got[keep] - want[keep]).max() <= 2e-2
    wk, wv = oracle.reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping)
    back = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    assert back(dc.k_cache).tobytes() == wk.tobytes()
    assert back(dc.v_cache).tobytes() == wv.tobytes()
