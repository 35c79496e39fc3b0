"""Pins for the CPU oracle: each test checks it against something other than
itself (a brute-force walk, a closed form, an invariant, a library routine or
the pages' worked figure), so that a dropped term, a wrong sign or index or a
transposed operand in the oracle fails at least one of them."""
import math
import os
import struct

import numpy as np
import pytest
import torch

import oracle
from oracle import oracle as O
from workloads import encode, gather_logical, layout_cache, make_case, assign_blocks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# independent helpers (pure Python; no oracle code)
# --------------------------------------------------------------------------
def py_value(bits, dtype):
    """Decode one stored scalar with struct, independently of the oracle."""
    if dtype == "f32":
        return float(bits)
    if dtype == "f16":
        return struct.unpack("<e", struct.pack("<H", int(bits)))[0]
    if dtype == "bf16":
        return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]
    raise ValueError(dtype)


def brute_decode(case):
    """Token-by-token walk of the block table with math.exp / math.tanh.

    The KV head of each query head comes from the widened list the X-Ray step
    draws (each KV head repeated G times, in order)."""
    B, Hq, D = case.q.shape
    Hkv, bs = case.Hkv, case.bs
    G = Hq // Hkv
    widened = [g for g in range(Hkv) for _ in range(G)]
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(case.context_lens[b])
        first = 0 if case.window <= 0 else max(0, L - case.window)
        for h in range(Hq):
            g = widened[h]
            qv = [py_value(case.q[b, h, d], case.dtype) for d in range(D)]
            scores, rows = [], []
            for t in range(first, L):
                phys = int(case.block_tables[b][t // bs])
                slot = t - (t // bs) * bs
                k = [py_value(case.k_cache[phys, slot, g, d], case.dtype) for d in range(D)]
                v = [py_value(case.v_cache[phys, slot, g, d], case.dtype) for d in range(D)]
                s = case.scale * sum(a * c for a, c in zip(qv, k))
                if case.softcap > 0:
                    s = case.softcap * math.tanh(s / case.softcap)
                scores.append(s)
                rows.append(v)
            if not scores:
                continue
            top = max(scores)
            w = [math.exp(s - top) for s in scores]
            tot = sum(w)
            for d in range(D):
                out[b, h, d] = sum(wi * r[d] for wi, r in zip(w, rows)) / tot
    return out


def small(dtype="f32", **kw):
    base = dict(B=3, Hq=4, Hkv=2, D=8, bs=4, dtype=dtype,
                context_lens=[1, 13, 27], seed=7)
    base.update(kw)
    return make_case(**base)


def run(case):
    return O.decode(case.q, case.k_cache, case.v_cache, case.block_tables,
                    case.context_lens, case.scale, case.softcap, case.window,
                    case.dtype)


# --------------------------------------------------------------------------
# storage decoding
# --------------------------------------------------------------------------
def test_decode_known_bit_patterns():
    bf = np.array([0x3F80, 0xC000, 0x3E20, 0x0000, 0x8000, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 0.15625, 0.0, -0.0, 3.140625]
    assert O.to_f64(bf, "bf16").tolist() == want
    hf = np.array([0x3C00, 0xC000, 0x3555, 0x7BFF], dtype=np.uint16)
    assert O.to_f64(hf, "f16").tolist() == [1.0, -2.0, 0.333251953125, 65504.0]


def test_encode_matches_torch_rounding():
    x = np.random.default_rng(0).standard_normal(4096).astype(np.float32) * 7
    ours = encode(x, "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    ours16 = encode(x, "f16")
    ref16 = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours16, ref16)


# --------------------------------------------------------------------------
# brute force on tiny inputs
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("softcap,window", [(0.0, 0), (3.0, 0), (0.0, 5), (2.0, 9)])
def test_brute_force_agrees(dtype, softcap, window):
    c = small(dtype, softcap=softcap, window=window, scale=0.7)
    got = run(c)
    want = brute_decode(c)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_brute_force_agrees_gqa8_bs1():
    c = make_case(B=2, Hq=16, Hkv=2, D=4, bs=1, dtype="bf16", context_lens=[5, 11],
                  seed=3, softcap=1.5)
    np.testing.assert_allclose(run(c), brute_decode(c), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_key_returns_v_exactly(dtype):
    c = small(dtype, context_lens=[1, 1, 1], softcap=50.0)
    got = run(c)
    for b in range(c.B):
        blk = c.block_tables[b, 0]
        for h in range(c.Hq):
            g = h // (c.Hq // c.Hkv)
            assert np.array_equal(got[b, h], O.to_f64(c.v_cache[blk, 0, g], dtype))


@pytest.mark.parametrize("softcap", [0.0, 50.0])
def test_identical_keys_give_mean_of_v(softcap):
    c = small("f32", context_lens=[5, 9, 16], softcap=softcap)
    for b in range(c.B):
        L = int(c.context_lens[b])
        first = c.k_cache[c.block_tables[b, 0], 0].copy()
        for t in range(L):
            c.k_cache[c.block_tables[b, t // c.bs], t % c.bs] = first
    got = run(c)
    for b in range(c.B):
        L = int(c.context_lens[b])
        rows = np.stack([c.v_cache[c.block_tables[b, t // c.bs], t % c.bs]
                         for t in range(L)]).astype(np.float64)
        mean = rows.mean(axis=0)  # [Hkv, D]
        G = c.Hq // c.Hkv
        np.testing.assert_allclose(got[b], np.repeat(mean, G, axis=0), rtol=0, atol=1e-12)


def test_window_one_returns_last_v():
    c = small("bf16", window=1, softcap=50.0)
    got = run(c)
    for b in range(c.B):
        t = int(c.context_lens[b]) - 1
        v = O.to_f64(c.v_cache[c.block_tables[b, t // c.bs], t % c.bs], "bf16")
        G = c.Hq // c.Hkv
        assert np.array_equal(got[b], np.repeat(v, G, axis=0))


def test_two_keys_softcap_closed_form():
    # one KV head, one query head, D = 2: logits reach the nonlinear part of tanh
    c = make_case(B=1, Hq=1, Hkv=1, D=2, bs=2, dtype="f32", context_lens=[2],
                  seed=1, scale=0.5, softcap=50.0, order="identity")
    c.q[0, 0] = [10.0, -4.0]
    c.k_cache[0, 0, 0] = [12.5, 0.25]    # scaled logit 62
    c.k_cache[0, 1, 0] = [11.0, 0.5]     # scaled logit 54
    c.v_cache[0, 0, 0] = [1.0, 2.0]
    c.v_cache[0, 1, 0] = [-5.0, 0.25]
    s1 = 50.0 * math.tanh(0.5 * (10 * 12.5 - 4 * 0.25) / 50.0)
    s2 = 50.0 * math.tanh(0.5 * (10 * 11.0 - 4 * 0.5) / 50.0)
    a = 1.0 / (1.0 + math.exp(s2 - s1))
    want = a * np.array([1.0, 2.0]) + (1 - a) * np.array([-5.0, 0.25])
    np.testing.assert_allclose(run(c)[0, 0], want, rtol=0, atol=1e-13)
    # and the cap is not a no-op here: without it the weights differ
    c0 = make_case(B=1, Hq=1, Hkv=1, D=2, bs=2, dtype="f32", context_lens=[2],
                   seed=1, scale=0.5, softcap=0.0, order="identity")
    c0.q[:], c0.k_cache[:], c0.v_cache[:] = c.q, c.k_cache, c.v_cache
    assert abs(run(c0)[0, 0, 0] - want[0]) > 1e-2


def test_huge_softcap_and_wide_window_reduce_to_plain():
    c = small("f32", scale=0.9)
    base = run(c)
    c.softcap = 1e12
    np.testing.assert_allclose(run(c), base, rtol=0, atol=1e-9)
    c.softcap = 0.0
    c.window = 10_000
    assert np.array_equal(run(c), base)


def test_textbook_attention_via_torch_sdpa():
    # G = 1, no cap, no window, identity block table -> dense softmax attention
    L = [6, 19, 32]
    c = make_case(B=3, Hq=3, Hkv=3, D=16, bs=8, dtype="f32", context_lens=L,
                  seed=11, order="identity", scale=0.31)
    got = run(c)
    for b in range(3):
        rows = gather_logical(c.k_cache, c.block_tables, c.context_lens)[b]
        vals = gather_logical(c.v_cache, c.block_tables, c.context_lens)[b]
        q = torch.from_numpy(c.q[b].astype(np.float64))[:, None, :]        # [H,1,D]
        k = torch.from_numpy(rows.astype(np.float64)).permute(1, 0, 2)      # [H,L,D]
        v = torch.from_numpy(vals.astype(np.float64)).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=0.31)
        np.testing.assert_allclose(got[b], ref[:, 0].numpy(), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------
def test_independent_of_block_size():
    c16 = small("bf16", bs=16, context_lens=[3, 40, 77], softcap=50.0, window=30)
    logical_k = gather_logical(c16.k_cache, c16.block_tables, c16.context_lens)
    logical_v = gather_logical(c16.v_cache, c16.block_tables, c16.context_lens)
    ref = run(c16)
    for bs in (1, 2, 32):
        rng = np.random.default_rng(bs)
        NB = sum((int(L) + bs - 1) // bs for L in c16.context_lens) + 5
        bt = assign_blocks(c16.context_lens, bs, NB, rng)
        kc = layout_cache(logical_k, bt, NB, bs, "bf16")
        vc = layout_cache(logical_v, bt, NB, bs, "bf16")
        got = O.decode(c16.q, kc, vc, bt, c16.context_lens, c16.scale, c16.softcap,
                       c16.window, "bf16")
        assert np.array_equal(got, ref)


def test_physical_block_permutation_is_invisible():
    c = small("f16", softcap=30.0)
    ref = run(c)
    perm = np.random.default_rng(5).permutation(c.NB)   # new id of old block i
    kc = np.empty_like(c.k_cache)
    vc = np.empty_like(c.v_cache)
    kc[perm] = c.k_cache
    vc[perm] = c.v_cache
    bt = np.where(c.block_tables >= 0, perm[np.maximum(c.block_tables, 0)], -1).astype(np.int32)
    got = O.decode(c.q, kc, vc, bt, c.context_lens, c.scale, c.softcap, c.window, "f16")
    assert np.array_equal(got, ref)


def test_token_permutation_is_invisible_without_window():
    c = small("f32", context_lens=[7, 20, 31], softcap=4.0)
    ref = run(c)
    lk = gather_logical(c.k_cache, c.block_tables, c.context_lens)
    lv = gather_logical(c.v_cache, c.block_tables, c.context_lens)
    rng = np.random.default_rng(9)
    for b in range(c.B):
        p = rng.permutation(lk[b].shape[0])
        lk[b], lv[b] = lk[b][p], lv[b][p]
    kc = layout_cache(lk, c.block_tables, c.NB, c.bs, "f32")
    vc = layout_cache(lv, c.block_tables, c.NB, c.bs, "f32")
    got = O.decode(c.q, kc, vc, c.block_tables, c.context_lens, c.scale, c.softcap, 0, "f32")
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_window_equals_last_w_tokens():
    c = small("f32", context_lens=[4, 17, 30], window=6, softcap=5.0)
    ref = run(c)
    lk = gather_logical(c.k_cache, c.block_tables, c.context_lens)
    lv = gather_logical(c.v_cache, c.block_tables, c.context_lens)
    tail_len = np.minimum(c.context_lens, 6)
    lk = [k[-n:] for k, n in zip(lk, tail_len)]
    lv = [v[-n:] for v, n in zip(lv, tail_len)]
    bt = assign_blocks(tail_len, c.bs, c.NB, np.random.default_rng(2))
    kc = layout_cache(lk, bt, c.NB, c.bs, "f32")
    vc = layout_cache(lv, bt, c.NB, c.bs, "f32")
    got = O.decode(c.q, kc, vc, bt, tail_len, c.scale, c.softcap, 0, "f32")
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_linear_in_v():
    c = small("f32", softcap=8.0)
    ref = run(c)
    a, s = -2.5, 0.75
    c.v_cache = (a * c.v_cache.astype(np.float64) + s).astype(np.float32)
    got = run(c)
    live = np.array(c.context_lens) > 0
    np.testing.assert_allclose(got[live], a * ref[live] + s, rtol=0, atol=1e-5)


def test_gqa_head_map():
    c = small("f32", Hq=8, Hkv=2, softcap=3.0)
    for g in range(c.Hkv):
        c.v_cache[:, :, g, :] = g + 1.0
    got = run(c)
    G = c.Hq // c.Hkv
    for h in range(c.Hq):
        np.testing.assert_allclose(got[:, h, :], h // G + 1.0, rtol=0, atol=1e-12)


def test_empty_context_gives_zero():
    c = small("f32", context_lens=[0, 5, 0])
    got = run(c)
    assert np.all(got[0] == 0) and np.all(got[2] == 0)


# --------------------------------------------------------------------------
# the pages' worked figures
# --------------------------------------------------------------------------
def read_fixture(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = v.split()
    return out


def test_pool_figure_layout_equals_contiguous():
    fx = read_fixture("paged_pool_figure.txt")
    NB = int(fx["pool_blocks"][0])
    A = [int(x) for x in fx["seq A"]]
    Bq = [int(x) for x in fx["seq B"]]
    free = [int(x) for x in fx["free"]]
    assert sorted(A + Bq + free) == list(range(NB))
    bs = 4
    L = [len(A) * bs - 1, len(Bq) * bs - 2]  # last blocks partly used
    contiguous = make_case(B=2, Hq=4, Hkv=2, D=8, bs=bs, dtype="bf16", context_lens=L,
                           NB=NB, order="identity", seed=21, softcap=50.0)
    lk = gather_logical(contiguous.k_cache, contiguous.block_tables, L)
    lv = gather_logical(contiguous.v_cache, contiguous.block_tables, L)
    bt = np.full((2, 3), -1, np.int32)
    bt[0, :2] = A
    bt[1, :3] = Bq
    kc = layout_cache(lk, bt, NB, bs, "bf16")   # free blocks and tails stay NaN
    vc = layout_cache(lv, bt, NB, bs, "bf16")
    assert np.isnan(O.to_f64(kc[free], "bf16")).all()
    got = O.decode(contiguous.q, kc, vc, bt, np.array(L), contiguous.scale, 50.0, 0, "bf16")
    assert np.isfinite(got).all()
    assert np.array_equal(got, run(contiguous))


def test_xray_gqa_shapes_and_scale():
    fx = read_fixture("xray_gqa_shapes.txt")
    Hq, Hkv, D, T = (int(fx[k][0]) for k in ("q_heads", "kv_heads", "head_dim", "tokens"))
    assert [int(x) for x in fx["scores_shape"]] == [1, Hq, T, T]
    scale = 1.0 / math.sqrt(int(fx["scale_denominator_sqrt_of"][0]))
    c = make_case(B=1, Hq=Hq, Hkv=Hkv, D=D, bs=16, dtype="f32", context_lens=[T],
                  seed=4, scale=scale)
    got = run(c)
    # the figure widens K to all query heads and multiplies Q by K^T
    K = gather_logical(c.k_cache, c.block_tables, [T])[0].astype(np.float64)   # [T,Hkv,D]
    V = gather_logical(c.v_cache, c.block_tables, [T])[0].astype(np.float64)
    Kw = np.repeat(K, Hq // Hkv, axis=1).transpose(1, 0, 2)                      # [Hq,T,D]
    Vw = np.repeat(V, Hq // Hkv, axis=1).transpose(1, 0, 2)
    Q = c.q[0].astype(np.float64)[:, None, :]                                    # [Hq,1,D]
    scores = Q @ Kw.transpose(0, 2, 1) / math.sqrt(D)                            # [Hq,1,T]
    w = np.exp(scores - scores.max(-1, keepdims=True))
    ref = (w @ Vw)[:, 0] / w.sum(-1)
    np.testing.assert_allclose(got[0], ref, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# reshape_and_cache
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_reshape_and_cache_scatter(dtype):
    rng = np.random.default_rng(3)
    NB, bs, Hkv, D, T = 6, 4, 2, 8, 9
    kc = encode(rng.standard_normal((NB, bs, Hkv, D)).astype(np.float32), dtype)
    vc = encode(rng.standard_normal((NB, bs, Hkv, D)).astype(np.float32), dtype)
    key = encode(rng.standard_normal((T, Hkv, D)).astype(np.float32), dtype)
    val = encode(rng.standard_normal((T, Hkv, D)).astype(np.float32), dtype)
    key[2, 1, 3] = np.float32(np.nan) if dtype == "f32" else np.uint16(0x7FC1)  # NaN payload
    slots = rng.choice(NB * bs, size=T, replace=False).astype(np.int64)
    slots[4] = -1
    nk, nv = O.reshape_and_cache(key, val, kc, vc, slots)
    want_k, want_v = kc.copy(), vc.copy()
    for i, s in enumerate(slots):
        if s < 0:
            continue
        blk, off = divmod(int(s), bs)
        want_k[blk, off] = key[i]
        want_v[blk, off] = val[i]
    assert nk.tobytes() == want_k.tobytes()
    assert nv.tobytes() == want_v.tobytes()


def test_reshape_and_cache_skips_slots_outside_the_pool():
    """Slots that name no slot of the pool (-1, other negatives, and every
    value >= num_blocks * block_size) leave both caches bit for bit as they
    were; the in-pool rows of the same call still land.  Checked against a
    slot-by-slot write of only the in-pool rows."""
    rng = np.random.default_rng(31)
    NB, bs, Hkv, D = 5, 4, 2, 8
    kc = encode(rng.standard_normal((NB, bs, Hkv, D)).astype(np.float32), "bf16")
    vc = encode(rng.standard_normal((NB, bs, Hkv, D)).astype(np.float32), "bf16")
    slots = np.array([NB * bs, 3, -1, NB * bs + 7, -5, 19, 2 ** 40], dtype=np.int64)
    key = encode(rng.standard_normal((len(slots), Hkv, D)).astype(np.float32), "bf16")
    val = encode(rng.standard_normal((len(slots), Hkv, D)).astype(np.float32), "bf16")
    nk, nv = O.reshape_and_cache(key, val, kc, vc, slots)
    want_k, want_v = kc.copy(), vc.copy()
    want_k[0, 3], want_v[0, 3] = key[1], val[1]      # slot 3
    want_k[4, 3], want_v[4, 3] = key[5], val[5]      # slot 19, the pool's last
    assert nk.tobytes() == want_k.tobytes()
    assert nv.tobytes() == want_v.tobytes()
    # only out-of-pool slots: nothing changes
    nk, nv = O.reshape_and_cache(key[:1], val[:1], kc, vc, slots[:1])
    assert nk.tobytes() == kc.tobytes() and nv.tobytes() == vc.tobytes()


# --------------------------------------------------------------------------
# planted mistakes: every mutant of the oracle must fail some pin above
# --------------------------------------------------------------------------
MUTANTS = {
    "head map h % Hkv": ("kv_head_of", lambda h, G: h % 2),
    "cap before scale": ("cap", lambda s, c: (c * np.tanh(s / c) * 1.1) if c > 0 else s),
    "flipped exponent sign": ("softmax_weighted_sum",
                              lambda s, V: (np.exp(s.min() - s) @ V) / np.exp(s.min() - s).sum()),
    "off-by-one window": ("attended_range",
                          lambda L, W: ((max(0, L - W - 1) if W > 0 else 0), L)),
    "dropped normaliser": ("softmax_weighted_sum", lambda s, V: np.exp(s - s.max()) @ V),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistakes_are_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    pins = [
        lambda: test_brute_force_agrees("f32", 3.0, 0),
        lambda: test_brute_force_agrees("f32", 0.0, 5),
        lambda: test_gqa_head_map(),
        lambda: test_two_keys_softcap_closed_form(),
        lambda: test_window_one_returns_last_v(),
    ]
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"mutant {name!r} survived every pin"


# --------------------------------------------------------------------------
# copy_blocks (copy-on-write of shared blocks)
# --------------------------------------------------------------------------
def test_copy_blocks_slot_by_slot():
    rng = np.random.default_rng(8)
    NB, bs, Hkv, D = 9, 4, 2, 8
    kc = encode(rng.standard_normal((NB, bs, Hkv, D)).astype(np.float32), "bf16")
    vc = encode(rng.standard_normal((NB, bs, Hkv, D)).astype(np.float32), "bf16")
    mapping = np.array([[0, 5], [3, 7], [12, 1], [2, -1]], dtype=np.int64)  # last two invalid
    nk, nv = O.copy_blocks(kc, vc, mapping)
    want_k, want_v = kc.copy(), vc.copy()
    for src, dst in [(0, 5), (3, 7)]:
        for t in range(bs):
            for g in range(Hkv):
                for d in range(D):
                    want_k[dst, t, g, d] = kc[src, t, g, d]
                    want_v[dst, t, g, d] = vc[src, t, g, d]
    assert nk.tobytes() == want_k.tobytes() and nv.tobytes() == want_v.tobytes()


def test_shared_prefix_blocks_decode_like_private_copies():
    """Two sequences whose tables point at the same physical prefix blocks
    attend exactly as if each owned a copy."""
    c = make_case(B=2, Hq=4, Hkv=2, D=8, bs=4, dtype="f32", context_lens=[10, 13],
                  seed=17, NB=12, order="identity")
    # sequence 1 reuses sequence 0's first two blocks (positions 0..7)
    shared = c.block_tables[0, :2].copy()
    own = c.block_tables[1, :2].copy()
    c.k_cache[own] = c.k_cache[shared]
    c.v_cache[own] = c.v_cache[shared]
    private = run(c)
    c.block_tables[1, :2] = shared
    assert np.array_equal(run(c), private)


# --------------------------------------------------------------------------
# multi-query attention (several new tokens per sequence, causal)
# --------------------------------------------------------------------------
from torch.nn.attention.bias import causal_lower_right  # noqa: E402

from workloads import make_mq_case  # noqa: E402


def widen_torch(bits, dtype):
    """Stored values -> float64 tensor via torch's own dtype conversions."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(bits)).double()
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).double()


def run_mq(c):
    return O.multi_query(c.q, c.query_start, c.k_cache, c.v_cache, c.block_tables,
                         c.context_lens, c.scale, c.softcap, c.window, c.dtype)


def sdpa_rows(c, b, mask):
    """Rows of sequence b by torch's scaled_dot_product_attention on the
    gathered keys, KV heads widened with repeat_interleave."""
    L = int(c.context_lens[b])
    G = c.Hq // c.Hkv
    K = widen_torch(gather_logical(c.k_cache, c.block_tables, c.context_lens)[b], c.dtype)
    V = widen_torch(gather_logical(c.v_cache, c.block_tables, c.context_lens)[b], c.dtype)
    q0, q1 = int(c.query_start[b]), int(c.query_start[b + 1])
    qb = widen_torch(c.q[q0:q1], c.dtype)                       # [n, Hq, D]
    K = K.repeat_interleave(G, dim=1).transpose(0, 1).contiguous()  # [Hq, L, D]
    V = V.repeat_interleave(G, dim=1).transpose(0, 1).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(
        qb.transpose(0, 1).contiguous(), K, V, attn_mask=mask(q1 - q0, L), scale=c.scale)
    return o.transpose(0, 1).numpy()


def mq_small(dtype="f32", **kw):
    base = dict(Hq=4, Hkv=2, D=8, bs=4, dtype=dtype, context_lens=[7, 13, 27, 5],
                query_lens=[3, 13, 6, 1], seed=23)
    base.update(kw)
    return make_mq_case(**base)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_mq_matches_sdpa_lower_right_causal(dtype):
    """New tokens are the last n positions: torch's bottom-right causal mask."""
    c = mq_small(dtype, scale=0.6)
    got = run_mq(c)
    for b in range(c.B):
        want = sdpa_rows(c, b, lambda n, L: causal_lower_right(n, L)._materialize())
        q0, q1 = c.query_start[b], c.query_start[b + 1]
        np.testing.assert_allclose(got[q0:q1], want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("W", [1, 4, 9])
def test_mq_window_matches_banded_sdpa(W):
    c = mq_small("bf16", window=W, scale=0.6)
    got = run_mq(c)

    def band(n, L):
        rows = torch.arange(L - n, L)[:, None]
        cols = torch.arange(L)[None, :]
        return (cols <= rows) & (cols > rows - W)

    for b in range(c.B):
        q0, q1 = c.query_start[b], c.query_start[b + 1]
        np.testing.assert_allclose(got[q0:q1], sdpa_rows(c, b, band), rtol=0, atol=1e-12)


def brute_mq(c):
    """Token-by-token walk with math.exp / math.tanh; every new token
    attends to the positions up to its own (window counted back from it)."""
    G = c.Hq // c.Hkv
    widened = [g for g in range(c.Hkv) for _ in range(G)]
    out = np.zeros((c.T, c.Hq, c.D))
    for b in range(c.B):
        L = int(c.context_lens[b])
        q0, q1 = int(c.query_start[b]), int(c.query_start[b + 1])
        for r in range(q0, q1):
            pos = L - (q1 - q0) + (r - q0)
            first = 0 if c.window <= 0 else max(0, pos + 1 - c.window)
            for h in range(c.Hq):
                g = widened[h]
                qv = [py_value(c.q[r, h, d], c.dtype) for d in range(c.D)]
                scores, rows = [], []
                for t in range(first, pos + 1):
                    phys = int(c.block_tables[b][t // c.bs])
                    slot = t - (t // c.bs) * c.bs
                    k = [py_value(c.k_cache[phys, slot, g, d], c.dtype) for d in range(c.D)]
                    v = [py_value(c.v_cache[phys, slot, g, d], c.dtype) for d in range(c.D)]
                    s = c.scale * sum(a * x for a, x in zip(qv, k))
                    if c.softcap > 0:
                        s = c.softcap * math.tanh(s / c.softcap)
                    scores.append(s)
                    rows.append(v)
                top = max(scores)
                w = [math.exp(s - top) for s in scores]
                tot = sum(w)
                for d in range(c.D):
                    out[r, h, d] = sum(wi * row[d] for wi, row in zip(w, rows)) / tot
    return out


@pytest.mark.parametrize("softcap,window", [(2.0, 0), (1.5, 6)])
def test_mq_brute_force_softcap_gqa(softcap, window):
    c = mq_small("bf16", Hq=8, Hkv=2, softcap=softcap, window=window, scale=0.9,
                 context_lens=[9, 14, 4], query_lens=[4, 14, 0])
    np.testing.assert_allclose(run_mq(c), brute_mq(c), rtol=0, atol=1e-12)


def test_mq_one_new_token_is_decode():
    c = mq_small("f16", query_lens=[1, 1, 1, 1], softcap=5.0, window=8)
    dec = O.decode(c.q, c.k_cache, c.v_cache, c.block_tables, c.context_lens, c.scale,
                   c.softcap, c.window, c.dtype)
    assert np.array_equal(run_mq(c), dec)


def test_mq_no_new_tokens():
    c = mq_small("f32", query_lens=[0, 0, 0, 0])
    assert run_mq(c).shape == (0, 4, 8)


def test_mq_last_row_sees_the_whole_context():
    """The newest token of a sequence attends to all of it, whatever the
    number of new tokens before it."""
    c = mq_small("bf16", query_lens=[7, 13, 1, 5], context_lens=[7, 13, 27, 5])
    got = run_mq(c)
    for b in range(c.B):
        last = int(c.query_start[b + 1]) - 1
        q1 = c.q[last][None]
        want = O.attend(q1[0], c.k_cache, c.v_cache, c.block_tables, b,
                        int(c.context_lens[b]), c.scale, 0.0, 0, c.dtype)
        assert np.array_equal(got[last], want)


MQ_MUTANTS = {
    "causal from the top": ("query_positions", lambda L, n: np.arange(0, n)),
    "causal off by one": ("query_positions", lambda L, n: np.arange(L - n - 1, L - 1)),
    "newest token first": ("query_positions", lambda L, n: np.arange(L - n, L)[::-1]),
}


@pytest.mark.parametrize("name", list(MQ_MUTANTS))
def test_mq_planted_mistakes_are_caught(name, monkeypatch):
    attr, fn = MQ_MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = 0
    for pin in (lambda: test_mq_matches_sdpa_lower_right_causal("f32"),
                lambda: test_mq_window_matches_banded_sdpa(4)):
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed += 1
    assert failed > 0, f"mutant {name!r} survived every pin"
