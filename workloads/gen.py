"""Seeded synthetic inputs for paged decode attention.

This module only *draws and lays out* inputs; it holds none of the attention
arithmetic.  Both the CPU oracle (through the tests and the bench's CPU leg)
and the GPU path consume exactly the arrays built here, so the two sides see
the same bits.

Storage convention (the "bits" both sides read):
  * ``f32``  -> ``np.float32`` arrays;
  * ``f16``  -> ``np.uint16`` arrays holding IEEE binary16 bit patterns;
  * ``bf16`` -> ``np.uint16`` arrays holding bfloat16 bit patterns.

Values are drawn as float32 N(0,1) and rounded to the storage dtype with
round-to-nearest-even.  The paged layout follows the statement of the problem
on the pages: a pool of fixed-size physical blocks ``[num_blocks, block_size,
kv_heads, head_dim]`` and a per-sequence block table of physical ids
(ovshake/nano-vllm README, "Key Concepts Explained: PagedAttention", the
B0..B7 pool figure; flex-nano-vllm README, file list: "page table and paged kv
cache").  Block ids are taken in order from a seeded permutation of the pool,
sequence by sequence, so logically adjacent blocks are physically scattered.
Slots that no sequence references (free blocks, the unused tail of a
sequence's last block, block-table padding) are filled with NaN (or -1 for
table padding) so that a kernel that reads them poisons its own output.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

DTYPES = ("f32", "f16", "bf16")
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
NAN_BITS = {"f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0)}


# --------------------------------------------------------------------------
# dtype encoding (input preparation only)
# --------------------------------------------------------------------------
def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype (RNE) and return its bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = x.view(np.uint32)
        # round to nearest even on the upper 16 bits; NaN stays a quiet NaN
        r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
             >> np.uint32(16)).astype(np.uint16)
        nan = np.isnan(x)
        if nan.any():
            r[nan] = NAN_BITS["bf16"]
        return r
    raise ValueError(f"unknown dtype {dtype!r}")


def storage_np_dtype(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


def poison_fill(shape, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.full(shape, np.nan, dtype=np.float32)
    return np.full(shape, NAN_BITS[dtype], dtype=np.uint16)


# --------------------------------------------------------------------------
# case description
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Case:
    name: str
    dtype: str
    q: np.ndarray              # [B, Hq, D] storage
    k_cache: np.ndarray        # [NB, bs, Hkv, D] storage (state before the new rows land)
    v_cache: np.ndarray
    block_tables: np.ndarray   # [B, max_blocks] int32, padding = -1
    context_lens: np.ndarray   # [B] int32, counts the new token
    scale: float
    softcap: float             # <= 0: off
    window: int                # <= 0: off
    partition_size: Optional[int]  # 0: one partition per sequence; None: library's choice
    key: Optional[np.ndarray] = None           # [T, Hkv, D] storage, new rows
    value: Optional[np.ndarray] = None
    slot_mapping: Optional[np.ndarray] = None  # [T] int64, -1 = skip

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def Hq(self):
        return self.q.shape[1]

    @property
    def D(self):
        return self.q.shape[2]

    @property
    def NB(self):
        return self.k_cache.shape[0]

    @property
    def bs(self):
        return self.k_cache.shape[1]

    @property
    def Hkv(self):
        return self.k_cache.shape[2]

    @property
    def max_blocks(self):
        return self.block_tables.shape[1]

    @property
    def max_context_len(self):
        return int(self.context_lens.max()) if self.B else 0

    def attended(self) -> np.ndarray:
        """Number of keys each sequence attends to (window applied)."""
        L = self.context_lens.astype(np.int64)
        if self.window > 0:
            return np.minimum(L, self.window)
        return L

    def algorithmic_bytes(self) -> dict:
        """Bytes the method itself must move for one layer-step.

        K and V rows of attended tokens, the query read and the output write,
        the block-table entries of the attended pages and the context lengths;
        plus the new rows read and written by reshape_and_cache.
        """
        eb = ELEM_BYTES[self.dtype]
        n = self.attended()
        L = self.context_lens.astype(np.int64)
        start = L - n
        pages = np.where(n > 0, (L - 1) // self.bs - start // self.bs + 1, 0)
        kv = int(n.sum()) * self.Hkv * self.D * eb * 2
        qo = 2 * self.B * self.Hq * self.D * eb
        meta = int(pages.sum()) * 4 + 4 * self.B
        rc = 0
        if self.slot_mapping is not None:
            T = self.slot_mapping.shape[0]
            rc = 2 * 2 * T * self.Hkv * self.D * eb + 8 * T
        return {"kv": kv, "q_out": qo, "meta": meta, "decode": kv + qo + meta,
                "reshape": rc, "total": kv + qo + meta + rc}


# --------------------------------------------------------------------------
# layout helpers
# --------------------------------------------------------------------------
def blocks_needed(context_lens: Sequence[int], bs: int) -> List[int]:
    return [(int(L) + bs - 1) // bs for L in context_lens]


def assign_blocks(context_lens, bs, NB, rng, order="shuffled"):
    """Block table from a pool of NB blocks: ids taken in order from a
    seeded permutation (or 0, 1, 2, ... for order='identity')."""
    need = blocks_needed(context_lens, bs)
    total = sum(need)
    if total > NB:
        raise ValueError(f"pool of {NB} blocks cannot hold {total}")
    pool = rng.permutation(NB) if order == "shuffled" else np.arange(NB)
    maxb = max(1, max(need) if need else 1)
    bt = np.full((len(need), maxb), -1, dtype=np.int32)
    at = 0
    for b, n in enumerate(need):
        bt[b, :n] = pool[at:at + n]
        at += n
    return bt


def layout_cache(logical: List[np.ndarray], block_tables: np.ndarray, NB: int,
                 bs: int, dtype: str, poison: bool = True) -> np.ndarray:
    """Scatter per-sequence rows [L_b, Hkv, D] into a paged pool."""
    Hkv, D = logical[0].shape[1:] if logical else (1, 1)
    cache = (poison_fill((NB, bs, Hkv, D), dtype) if poison
             else np.zeros((NB, bs, Hkv, D), dtype=storage_np_dtype(dtype)))
    for b, rows in enumerate(logical):
        L = rows.shape[0]
        if L == 0:
            continue
        pos = np.arange(L)
        cache[block_tables[b, pos // bs], pos % bs] = rows
    return cache


def gather_logical(cache: np.ndarray, block_tables: np.ndarray, context_lens) -> List[np.ndarray]:
    """Inverse of layout_cache (used by tests to re-lay the same data)."""
    bs = cache.shape[1]
    out = []
    for b, L in enumerate(context_lens):
        pos = np.arange(int(L))
        out.append(cache[block_tables[b, pos // bs], pos % bs].copy())
    return out


# --------------------------------------------------------------------------
# generic builder
# --------------------------------------------------------------------------
def make_case(*, B: int, Hq: int, Hkv: int, D: int, bs: int, dtype: str,
              context_lens: Sequence[int], NB: Optional[int] = None,
              scale: Optional[float] = None, softcap: float = 0.0,
              window: int = 0, partition_size: Optional[int] = 0, seed: int = 0,
              new_rows: bool = False, poison: bool = True,
              order: str = "shuffled", name: str = "custom",
              extra_table_cols: int = 0) -> Case:
    """Build a synthetic case.  Streams of SeedSequence(seed).spawn(5):
    0 context lengths (unused here: lengths are given), 1 block permutation,
    2 q, 3 K/V rows, 4 new rows."""
    assert dtype in DTYPES
    context_lens = np.asarray(context_lens, dtype=np.int32)
    assert context_lens.shape == (B,)
    ss = np.random.SeedSequence(seed).spawn(5)
    r_perm, r_q, r_kv, r_new = (np.random.default_rng(s) for s in ss[1:])
    need = sum(blocks_needed(context_lens, bs))
    if NB is None:
        NB = max(1, int(need * 1.1) + 1)
    bt = assign_blocks(context_lens, bs, NB, r_perm, order)
    if extra_table_cols:
        bt = np.concatenate([bt, np.full((B, extra_table_cols), -1, np.int32)], axis=1)
    q = encode(r_q.standard_normal((B, Hq, D), dtype=np.float32), dtype)

    sdt = storage_np_dtype(dtype)
    kc = (poison_fill((NB, bs, Hkv, D), dtype) if poison
          else np.zeros((NB, bs, Hkv, D), dtype=sdt))
    vc = kc.copy()
    for b in range(B):
        L = int(context_lens[b])
        if L == 0:
            continue
        pos = np.arange(L)
        blk, off = bt[b, pos // bs], pos % bs
        kc[blk, off] = encode(r_kv.standard_normal((L, Hkv, D), dtype=np.float32), dtype)
        vc[blk, off] = encode(r_kv.standard_normal((L, Hkv, D), dtype=np.float32), dtype)

    key = value = slots = None
    if new_rows:
        # one new token per sequence, at its last position L-1: its slot is
        # poisoned here and filled by reshape_and_cache
        live = [b for b in range(B) if context_lens[b] > 0]
        T = len(live)
        key = encode(r_new.standard_normal((T, Hkv, D), dtype=np.float32), dtype)
        value = encode(r_new.standard_normal((T, Hkv, D), dtype=np.float32), dtype)
        slots = np.empty(T, dtype=np.int64)
        for i, b in enumerate(live):
            p = int(context_lens[b]) - 1
            blk, off = int(bt[b, p // bs]), p % bs
            slots[i] = blk * bs + off
            kc[blk, off] = poison_fill((Hkv, D), dtype)
            vc[blk, off] = poison_fill((Hkv, D), dtype)

    if scale is None:
        scale = 1.0 / float(np.sqrt(D))
    return Case(name=name, dtype=dtype, q=q, k_cache=kc, v_cache=vc,
                block_tables=bt, context_lens=context_lens, scale=float(scale),
                softcap=float(softcap), window=int(window),
                partition_size=partition_size, key=key, value=value,
                slot_mapping=slots)


# --------------------------------------------------------------------------
# the five named workloads
# --------------------------------------------------------------------------
WORKLOADS = {
    1: "tiny-f32-gqa4-d64",
    2: "gemma2-2b-global-bf16-b64",
    3: "gemma2-2b-sliding-bf16-b16",
    4: "gemma2-2b-serving-bf16-b512",
    5: "llama-gqa8-long-f16-b33",
}


def workload_lengths(n: int) -> np.ndarray:
    """Context lengths of workload n, from stream 0 of SeedSequence(1000+n)."""
    r = np.random.default_rng(np.random.SeedSequence(1000 + n).spawn(5)[0])
    if n == 1:
        return np.array([17, 64, 100, 255], dtype=np.int32)
    if n == 2:
        return r.integers(128, 1024, size=64, endpoint=True).astype(np.int32)
    if n == 3:
        return r.integers(4096, 8192, size=16, endpoint=True).astype(np.int32)
    if n == 4:
        prompt = r.integers(16, 512, size=512, endpoint=True)
        gen = r.integers(1, 512, size=512, endpoint=True)
        return (prompt + gen).astype(np.int32)
    if n == 5:
        L = r.integers(8192, 32768, size=32, endpoint=True)
        return np.concatenate([L, [131072]]).astype(np.int32)
    raise ValueError(n)


def workload(n: int, poison: bool = True, partition_size: Optional[int] = None) -> Case:
    """Workload n (1..5) at its full size.  Workloads 1, 3 and 5 fix their
    split (none; 512 tokens; 512 tokens); 2 and 4 leave it to the library
    (None) unless ``partition_size`` is given."""
    L = workload_lengths(n)
    seed = 1000 + n
    if n == 1:
        c = make_case(B=4, Hq=8, Hkv=2, D=64, bs=16, dtype="f32", context_lens=L,
                      NB=64, scale=1 / 8, seed=seed, poison=poison,
                      partition_size=0 if partition_size is None else partition_size)
    elif n == 2:
        c = make_case(B=64, Hq=8, Hkv=4, D=256, bs=16, dtype="bf16", context_lens=L,
                      NB=8192, scale=1 / 16, softcap=50.0, seed=seed, new_rows=True,
                      poison=poison, partition_size=partition_size)
    elif n == 3:
        c = make_case(B=16, Hq=8, Hkv=4, D=256, bs=16, dtype="bf16", context_lens=L,
                      scale=1 / 16, softcap=50.0, window=4096, seed=seed, poison=poison,
                      partition_size=512 if partition_size is None else partition_size)
    elif n == 4:
        c = make_case(B=512, Hq=8, Hkv=4, D=256, bs=16, dtype="bf16", context_lens=L,
                      NB=40000, scale=1 / 16, softcap=50.0, seed=seed, poison=poison,
                      new_rows=True, partition_size=partition_size)
    elif n == 5:
        c = make_case(B=33, Hq=32, Hkv=4, D=64, bs=32, dtype="f16", context_lens=L,
                      scale=1 / 8, seed=seed, poison=poison,
                      partition_size=512 if partition_size is None else partition_size)
    else:
        raise ValueError(n)
    c.name = WORKLOADS[n]
    return c


# --------------------------------------------------------------------------
# multi-query cases: several new tokens per sequence
# --------------------------------------------------------------------------
@dataclasses.dataclass
class MQCase:
    name: str
    dtype: str
    q: np.ndarray              # [T, Hq, D] storage, tokens packed sequence by sequence
    query_start: np.ndarray    # [B+1] int32: sequence b owns rows query_start[b] .. [b+1]-1
    k_cache: np.ndarray        # [NB, bs, Hkv, D] storage (state before the new rows land)
    v_cache: np.ndarray
    block_tables: np.ndarray   # [B, max_blocks] int32
    context_lens: np.ndarray   # [B] int32, counts every new token
    scale: float
    softcap: float
    window: int
    partition_size: Optional[int]
    key: Optional[np.ndarray] = None           # [T, Hkv, D] new rows of the new tokens
    value: Optional[np.ndarray] = None
    slot_mapping: Optional[np.ndarray] = None  # [T] int64

    @property
    def B(self):
        return self.context_lens.shape[0]

    @property
    def T(self):
        return self.q.shape[0]

    @property
    def Hq(self):
        return self.q.shape[1]

    @property
    def D(self):
        return self.q.shape[2]

    @property
    def NB(self):
        return self.k_cache.shape[0]

    @property
    def bs(self):
        return self.k_cache.shape[1]

    @property
    def Hkv(self):
        return self.k_cache.shape[2]

    @property
    def query_lens(self):
        return np.diff(self.query_start.astype(np.int64))

    @property
    def max_context_len(self):
        return int(self.context_lens.max()) if self.B else 0

    @property
    def max_query_len(self):
        return int(self.query_lens.max()) if self.B else 0

    def algorithmic_bytes(self) -> dict:
        """K/V rows of the union of the keys a sequence's new tokens attend
        to (read once), q read + out write, table entries, lengths and
        offsets; plus the new rows written by reshape_and_cache."""
        eb = ELEM_BYTES[self.dtype]
        L = self.context_lens.astype(np.int64)
        n = self.query_lens
        first = L - n  # position of the first new token
        lo = np.maximum(0, first + 1 - self.window) if self.window > 0 else np.zeros_like(L)
        keys = np.where(n > 0, L - lo, 0)
        pages = np.where(n > 0, (L - 1) // self.bs - lo // self.bs + 1, 0)
        kv = int(keys.sum()) * self.Hkv * self.D * eb * 2
        qo = 2 * self.T * self.Hq * self.D * eb
        meta = int(pages.sum()) * 4 + 4 * self.B + 4 * (self.B + 1)
        rc = 0
        if self.slot_mapping is not None:
            rc = 2 * 2 * self.T * self.Hkv * self.D * eb + 8 * self.T
        return {"kv": kv, "q_out": qo, "meta": meta, "attn": kv + qo + meta,
                "reshape": rc, "total": kv + qo + meta + rc}

    def flops(self) -> int:
        """4 * D flops (q.k and p.v) per (query head, attended key) pair."""
        L = self.context_lens.astype(np.int64)
        tot = 0
        for b in range(self.B):
            n = int(self.query_lens[b])
            pos = np.arange(L[b] - n, L[b])
            keys = pos + 1 if self.window <= 0 else np.minimum(pos + 1, self.window)
            tot += int(keys.sum())
        return 4 * self.D * self.Hq * tot


def make_mq_case(*, Hq: int, Hkv: int, D: int, bs: int, dtype: str,
                 context_lens: Sequence[int], query_lens: Sequence[int],
                 NB: Optional[int] = None, scale: Optional[float] = None,
                 softcap: float = 0.0, window: int = 0,
                 partition_size: Optional[int] = 0, seed: int = 0,
                 new_rows: bool = False, poison: bool = True,
                 order: str = "shuffled", name: str = "custom-mq") -> MQCase:
    """A multi-query case: sequence b holds context_lens[b] tokens, of which
    the last query_lens[b] are new (their queries are q's rows, in position
    order).  The cache comes from ``make_case`` with the same seed; q and the
    new rows are drawn from streams 5 and 6 of SeedSequence(seed).spawn(7)."""
    L = np.asarray(context_lens, dtype=np.int32)
    n = np.asarray(query_lens, dtype=np.int32)
    assert L.shape == n.shape and (n <= L).all() and (n >= 0).all()
    B = L.shape[0]
    base = make_case(B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs, dtype=dtype, context_lens=L, NB=NB,
                     scale=scale, softcap=softcap, window=window,
                     partition_size=partition_size, seed=seed, poison=poison, order=order)
    ss = np.random.SeedSequence(seed).spawn(7)
    r_q, r_new = np.random.default_rng(ss[5]), np.random.default_rng(ss[6])
    qs = np.zeros(B + 1, dtype=np.int32)
    qs[1:] = np.cumsum(n)
    T = int(qs[-1])
    q = encode(r_q.standard_normal((T, Hq, D), dtype=np.float32), dtype)
    kc, vc = base.k_cache, base.v_cache
    key = value = slots = None
    if new_rows:
        key = encode(r_new.standard_normal((T, Hkv, D), dtype=np.float32), dtype)
        value = encode(r_new.standard_normal((T, Hkv, D), dtype=np.float32), dtype)
        slots = np.empty(T, dtype=np.int64)
        for b in range(B):
            for i in range(int(n[b])):
                pos = int(L[b]) - int(n[b]) + i
                blk, off = int(base.block_tables[b, pos // bs]), pos % bs
                slots[qs[b] + i] = blk * bs + off
                kc[blk, off] = poison_fill((Hkv, D), dtype)
                vc[blk, off] = poison_fill((Hkv, D), dtype)
    return MQCase(name=name, dtype=dtype, q=q, query_start=qs, k_cache=kc, v_cache=vc,
                  block_tables=base.block_tables, context_lens=L, scale=base.scale,
                  softcap=base.softcap, window=base.window, partition_size=partition_size,
                  key=key, value=value, slot_mapping=slots)


MQ_WORKLOADS = {
    "spec5": "gemma2-2b-spec-verify5-bf16-b512",
    "chunk512": "gemma2-2b-chunked-prefill512-bf16",
    "prefill": "llama-gqa8-prefill-f16",
}


def mq_workload(name: str, poison: bool = True,
                partition_size: Optional[int] = None) -> MQCase:
    """Named multi-query workloads at full size.

    spec5    the Gemma-2 serving batch of workload 4 (512 sequences, lengths
             17..1024) verifying 5 speculative tokens each (the pages'
             speculative-decoding example uses 5);
    chunk512 one 512-token chunk of a 4096-token Gemma-2 prompt (the pages'
             default chunked-prefill budget is 512 tokens) batched with 63
             decoding sequences of workload 2's lengths;
    prefill  4 prompts of 2048 tokens each, prefilled whole (f16, 32/4
             heads, head_dim 64, block 32), every K/V row landing in the
             cache first."""
    if name == "spec5":
        L = workload_lengths(4)
        n = np.full(L.shape, 5, dtype=np.int32)
        L = np.maximum(L, 5)
        c = make_mq_case(Hq=8, Hkv=4, D=256, bs=16, dtype="bf16", context_lens=L,
                         query_lens=n, NB=40000, scale=1 / 16, softcap=50.0, seed=1101,
                         poison=poison, new_rows=True, partition_size=partition_size)
    elif name == "chunk512":
        Ld = workload_lengths(2)[:63]
        L = np.concatenate([[4096], Ld]).astype(np.int32)
        n = np.concatenate([[512], np.ones(63, dtype=np.int32)]).astype(np.int32)
        c = make_mq_case(Hq=8, Hkv=4, D=256, bs=16, dtype="bf16", context_lens=L,
                         query_lens=n, NB=8192, scale=1 / 16, softcap=50.0, seed=1102,
                         poison=poison, new_rows=True, partition_size=partition_size)
    elif name == "prefill":
        L = np.full(4, 2048, dtype=np.int32)
        c = make_mq_case(Hq=32, Hkv=4, D=64, bs=32, dtype="f16", context_lens=L,
                         query_lens=L, scale=1 / 8, seed=1103, poison=poison,
                         new_rows=True, partition_size=partition_size)
    else:
        raise ValueError(name)
    c.name = MQ_WORKLOADS[name]
    return c
