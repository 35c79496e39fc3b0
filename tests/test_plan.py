"""The work plans, read back from the workspace after a GPU call.

Outputs alone cannot show that a plan lists each piece of work once: a unit
run twice writes the same values twice.  These tests read the plans the
launches used (their place in the workspace is the layout documented for
pa_decode_workspace_size and pa_mq_workspace_size) and check them against
the shapes: the decode plan's sequence order is a permutation, longest
first; the multi-query plan's row tiles cover every sequence's rows once,
the most keys first, and (keys split, workgroup-shared kernel) its unit list
holds every (tile, partition) that has keys exactly once, the most work
first.  Order is checked to within one of the plan's 256 buckets."""
import os

import numpy as np
import pytest

from workloads import make_case, make_mq_case

pytestmark = pytest.mark.gpu

NBK = 256


def pad(x):
    return (x + 255) // 256 * 256


def bucket(work, of):
    """The plan's bucket of `work` out of `of` (0 holds the most), exact."""
    return NBK - 1 - min(NBK - 1, max(work, 0) * (NBK - 1) // of)


def assert_bucket_order(works, of):
    b = [bucket(w, of) for w in works]
    bad = [i for i in range(len(b) - 1) if b[i] > b[i + 1] + 1]
    assert not bad, f"out of order at {bad[:5]}: {[(works[i], works[i + 1]) for i in bad[:5]]}"


def mq_max_tiles(B, T, G, R):
    rows = T * G
    return min(rows // R + B, rows)


@pytest.mark.parametrize("P,W", [(64, 0), (64, 100), (48, 20)])
def test_mq_plan_tiles_and_units(P, W):
    import torch
    import paged_kv_decode_pa_amd as pa
    from gpu_util import say, upload
    say(f"mq plan P={P} W={W}")
    rng = np.random.default_rng(2300 + P + W)
    L = [700, 1, 300, 64, 0, 1200, 33, 500, 90, 257]
    n = [96, 1, 1, 64, 0, 1, 5, 1, 40, 1]
    Hq, Hkv, D = 8, 4, 256
    G = Hq // Hkv
    c = make_mq_case(Hq=Hq, Hkv=Hkv, D=D, bs=16, dtype="bf16", context_lens=L, query_lens=n,
                     softcap=50.0, window=W, partition_size=P, seed=int(rng.integers(1 << 30)),
                     new_rows=True)
    B, T = len(L), int(sum(n))
    q = upload(c.q, "bf16")
    kc, vc = upload(c.k_cache, "bf16"), upload(c.v_cache, "bf16")
    bt = torch.from_numpy(c.block_tables).cuda()
    cl = torch.from_numpy(c.context_lens).cuda()
    qs = torch.from_numpy(c.query_start).cuda()
    maxL = int(c.max_context_len)
    nbytes = pa.mq_workspace_size(B, T, Hq, Hkv, D, maxL, P)
    ws = torch.zeros((nbytes + 3) // 4, dtype=torch.int32, device="cuda")
    os.environ["PA_MQ_WG"] = "1"
    try:
        pa.mq_attention(q, qs, kc, vc, bt, cl, c.scale, c.softcap, W, partition_size=P,
                        max_context_len=maxL, max_query_len=max(n), workspace=ws.view(torch.float32))
        torch.cuda.synchronize()
    finally:
        os.environ.pop("PA_MQ_WG")
    w = ws.cpu().numpy()
    R = 64  # head_dim 256: one 16-row block per wavefront, four wavefronts
    off_tiles = 2 * pad(T * 4)
    off_cnt = off_tiles + pad(mq_max_tiles(B, T, G, 16) * 8)
    ntiles, nunits = int(w[off_cnt // 4]), int(w[off_cnt // 4 + 1])
    tiles = w[off_tiles // 4: off_tiles // 4 + 2 * ntiles].reshape(-1, 2)
    units = w[(off_cnt + 256) // 4: (off_cnt + 256) // 4 + 2 * nunits].reshape(-1, 2)

    def span(b, f0):
        first = L[b] - n[b] + f0 // G
        khi = L[b] - n[b] + (min(f0 + R, n[b] * G) - 1) // G + 1
        klo = max(0, first + 1 - W) if W > 0 else 0
        return klo, khi

    want_tiles = sorted((b, f0) for b in range(B) for f0 in range(0, n[b] * G, R))
    assert sorted(map(tuple, tiles.tolist())) == want_tiles
    assert_bucket_order([min(max(span(b, f0)[1] - span(b, f0)[0], 0), maxL)
                         for b, f0 in tiles.tolist()], maxL)

    want_units, work = [], {}
    for i, (b, f0) in enumerate(tiles.tolist()):
        klo, khi = span(b, f0)
        waves = min((min(R, n[b] * G - f0) + R // 4 - 1) // (R // 4), 4)
        part = klo // P
        while part * P < khi and klo < khi:
            want_units.append((i, part))
            work[(i, part)] = (min(khi, part * P + P) - max(klo, part * P)) * waves
            part += 1
    got = list(map(tuple, units.tolist()))
    assert len(got) == len(set(got)), "a unit listed twice"
    assert sorted(got) == sorted(want_units)
    assert_bucket_order([work[u] for u in got], 4 * P)


def test_decode_plan_order_is_longest_first():
    """100 sequences over 4 KV heads (400 workgroups, more than the CUs): the
    launch takes the plan's order, longest first."""
    import torch
    import paged_kv_decode_pa_amd as pa
    from gpu_util import DeviceCase, say
    say("decode plan order")
    rng = np.random.default_rng(2400)
    L = rng.integers(1, 900, size=100).astype(np.int32)
    c = make_case(B=len(L), Hq=8, Hkv=4, D=128, bs=16, dtype="bf16", context_lens=L,
                  partition_size=0, seed=2401)
    dc = DeviceCase(c)
    maxL = int(L.max())
    nbytes = pa.workspace_size(len(L), 8, 128, maxL, 0)
    ws = torch.full(((nbytes + 3) // 4,), -7, dtype=torch.int32, device="cuda")
    out = torch.empty_like(dc.q)
    pa.decode_partitions(out, ws.view(torch.float32), dc.q, dc.k_cache, dc.v_cache,
                         dc.block_tables, dc.context_lens, maxL, c.scale, c.softcap, 0, 0)
    torch.cuda.synchronize()
    order = ws[:len(L)].cpu().numpy()
    assert sorted(order.tolist()) == list(range(len(L)))
    assert_bucket_order([int(L[b]) for b in order], maxL)
