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
