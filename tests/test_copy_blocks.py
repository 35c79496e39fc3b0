"""Block sharing on the GPU: pa_copy_blocks is bit-exact against the oracle's
copy, and the copy-on-write flow of a shared prefix (two sequences on the same
physical blocks, one appends a token after copying the partly filled shared
block) decodes like the oracle for both sequences."""
import numpy as np
import pytest

import oracle
from workloads import encode, make_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,D,bs,Hkv", [("bf16", 256, 16, 4), ("f16", 64, 32, 4),
                                             ("f32", 128, 1, 2)])
def test_copy_blocks_bit_exact(dtype, D, bs, Hkv):
    import torch
    import paged_kv_decode_pa_amd as pa
    from gpu_util import say, upload
    say(f"copy_blocks {dtype} D={D} bs={bs}")
    rng = np.random.default_rng(D + bs)
    NB = 40
    kc = encode(rng.standard_normal((NB, bs, Hkv, D)).astype(np.float32), dtype)
    vc = encode(rng.standard_normal((NB, bs, Hkv, D)).astype(np.float32), dtype)
    perm = rng.permutation(NB)
    mapping = np.stack([perm[:10], perm[10:20]], axis=1).astype(np.int64)
    mapping[3] = [NB + 5, 1]   # skipped: source outside the pool
    dk, dv = upload(kc, dtype), upload(vc, dtype)
    pa.copy_blocks(dk, dv, torch.from_numpy(mapping).cuda())
    torch.cuda.synchronize()
    back = lambda t: (t.view(torch.int16).cpu().numpy().view(np.uint16)
                      if dtype != "f32" else t.cpu().numpy())
    wk, wv = oracle.copy_blocks(kc, vc, mapping)
    assert back(dk).tobytes() == wk.tobytes()
    assert back(dv).tobytes() == wv.tobytes()


def test_copy_on_write_of_a_shared_prefix():
    import torch
    import paged_kv_decode_pa_amd as pa
    from gpu_util import DeviceCase, say, to_f64, upload
    say("copy on write")
    bs = 16
    # sequence 0 holds 40 tokens in 3 blocks (last one partly filled); sequence
    # 1 shares all three blocks (same prompt) and appends its own token at 40
    c = make_case(B=2, Hq=8, Hkv=4, D=256, bs=bs, dtype="bf16", context_lens=[40, 40],
                  softcap=50.0, seed=41, NB=16)
    c.block_tables[1, :3] = c.block_tables[0, :3]
    dc = DeviceCase(c)
    free_block = int(np.setdiff1d(np.arange(c.NB), c.block_tables[0, :3])[0])
    # copy-on-write: sequence 1 gets a private copy of the shared last block
    last = int(c.block_tables[0, 2])
    mapping = np.array([[last, free_block]], dtype=np.int64)
    pa.copy_blocks(dc.k_cache, dc.v_cache, torch.from_numpy(mapping).cuda())
    c.k_cache, c.v_cache = oracle.copy_blocks(c.k_cache, c.v_cache, mapping)
    c.block_tables[1, 2] = free_block
    dc.block_tables.copy_(torch.from_numpy(c.block_tables))
    shared_k = dc.k_cache[last].clone()
    # sequence 1 appends token 40 into its private block
    rng = np.random.default_rng(3)
    key = encode(rng.standard_normal((1, 4, 256)).astype(np.float32), "bf16")
    val = encode(rng.standard_normal((1, 4, 256)).astype(np.float32), "bf16")
    slots = np.array([free_block * bs + 40 % bs], dtype=np.int64)
    pa.reshape_and_cache(upload(key, "bf16"), upload(val, "bf16"), dc.k_cache, dc.v_cache,
                         torch.from_numpy(slots).cuda())
    c.k_cache, c.v_cache = oracle.reshape_and_cache(key, val, c.k_cache, c.v_cache, slots)
    c.context_lens = np.array([40, 41], dtype=np.int32)
    dc.context_lens.copy_(torch.from_numpy(c.context_lens))
    got = to_f64(pa.decode(dc.q, dc.k_cache, dc.v_cache, dc.block_tables, dc.context_lens,
                           c.scale, c.softcap, partition_size=0, max_context_len=41))
    want = oracle.decode(c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, c.scale,
                         c.softcap, 0, "bf16")
    assert np.isfinite(got).all() and np.abs(got - want).max() <= 2e-2
    # the append went to the private copy: the shared block is untouched
    assert torch.equal(dc.k_cache[last].view(torch.int16), shared_k.view(torch.int16))
