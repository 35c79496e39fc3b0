"""CPU oracle for paged attention: one new query token per sequence (decode)
or several (multi-query, causal among the new tokens).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code
with the GPU library and imports nothing from it.

It computes the plain definition, the simplest way: for each sequence, gather
its pages into contiguous K/V ("batch gathering", MinivLLM summary on
sourcepulse, "Highlighted Details"), widen every stored value exactly to
float64, and evaluate dense softmax attention of the one new query token
against the attended keys.

Definitions followed:
  * scores = q . k / sqrt(d) with the caller's scale (ovshake/nano-vllm README,
    "X-Ray Mode", Step 2 "Compute Attention Scores");
  * grouped-query attention: query head h reads KV head floor(h / G), G =
    Hq / Hkv, i.e. the KV heads repeated G times in order, as the same step
    shows K widened from 8 to 32 heads (same README, "X-Ray Mode", Step 1 GQA
    note and Step 2 shapes);
  * the page table: logical block j of a sequence lives in physical block
    block_tables[b][j], token t at slot t % block_size (same README, "Key
    Concepts Explained: PagedAttention"; flex-nano-vllm README, file list);
  * decode processes only the new token, so there is one query per sequence
    and its keys are positions [0, L) with L counting the new token (same
    README, "Key Concepts Explained: KV Cache");
  * several new tokens per sequence (chunked prefill, speculative
    verification: ovshake/nano-vllm README, "Features", "Advanced Scheduling"
    and "Optimizations") are causal: each sees the keys up to its own
    position (the self-attention chapter under that README's "Educational
    Modes", on the triangular mask);
  * Gemma-2 logit soft-capping s -> c * tanh(s / c), applied after scaling,
    and a sliding window keeping the last W keys [max(0, L - W), L): the
    pages name Gemma 2 (flex-nano-vllm README, opening line) but print
    neither rule; this is the public Gemma-2 attention definition (reading).
"""
from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------
# exact widening of stored values
# --------------------------------------------------------------------------
def to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored values to float64 exactly."""
    if dtype == "f32":
        return np.asarray(bits, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# reshape_and_cache: scatter new rows into their physical slots
# --------------------------------------------------------------------------
def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping):
    """Return copies of the caches with row i of key/value written at slot
    slot_mapping[i] (slot = physical_block * block_size + offset).  Only the
    new token's row is written (ovshake/nano-vllm README, "Key Concepts
    Explained: KV Cache").  A slot that names no slot of the pool -- -1, the
    usual "no slot" mark, or any value outside [0, num_blocks * block_size)
    -- is skipped (reading: the pages define no such slot; the library's
    contract for it is to leave the caches untouched).  Pure bit copies: the
    result is exact."""
    kc = k_cache.copy()
    vc = v_cache.copy()
    NB, bs, Hkv, D = kc.shape
    kf = kc.reshape(NB * bs, Hkv, D)
    vf = vc.reshape(NB * bs, Hkv, D)
    for i, s in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if s < 0 or s >= NB * bs:
            continue
        kf[s] = key[i]
        vf[s] = value[i]
    return kc, vc


def copy_blocks(k_cache, v_cache, block_mapping):
    """Return copies of the caches with whole block dst replaced by block src
    for each (src, dst) pair (the copy-on-write of a shared block); pairs with
    an id outside the pool are skipped.  Bit copies."""
    kc = k_cache.copy()
    vc = v_cache.copy()
    NB = kc.shape[0]
    for src, dst in np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2):
        if 0 <= src < NB and 0 <= dst < NB:
            kc[dst] = k_cache[src]
            vc[dst] = v_cache[src]
    return kc, vc


# --------------------------------------------------------------------------
# decode attention
# --------------------------------------------------------------------------
def attended_range(L: int, window: int):
    """Keys a decode query attends to: [start, L)."""
    start = max(0, L - window) if window > 0 else 0
    return start, L


def gather_sequence(cache, block_tables, b, start, L, dtype):
    """Contiguous float64 rows [n, Hkv, D] of positions [start, L) of seq b."""
    bs = cache.shape[1]
    pos = np.arange(start, L)
    blk = block_tables[b, pos // bs]
    off = pos % bs
    return to_f64(cache[blk, off], dtype)


def kv_head_of(h: int, G: int) -> int:
    return h // G


def cap(s: np.ndarray, softcap: float) -> np.ndarray:
    if softcap > 0:
        return softcap * np.tanh(s / softcap)
    return s


def softmax_weighted_sum(s: np.ndarray, V: np.ndarray) -> np.ndarray:
    """sum_t softmax(s)_t V[t], with the maximum subtracted for range."""
    p = np.exp(s - s.max())
    return (p @ V) / p.sum()


def attend(q_row, k_cache, v_cache, block_tables, b, L, scale, softcap, window,
           dtype):
    """float64 output [Hq, D] of one query token q_row [Hq, D] of sequence b
    whose context is the sequence's positions [0, L) (window applied)."""
    Hq, D = q_row.shape
    Hkv = k_cache.shape[2]
    G = Hq // Hkv
    out = np.zeros((Hq, D), dtype=np.float64)
    if L <= 0:
        return out
    start, end = attended_range(L, window)
    K = gather_sequence(k_cache, block_tables, b, start, end, dtype)
    V = gather_sequence(v_cache, block_tables, b, start, end, dtype)
    qb = to_f64(q_row, dtype)
    for h in range(Hq):
        g = kv_head_of(h, G)
        s = scale * (K[:, g, :] @ qb[h])
        s = cap(s, softcap)
        out[h] = softmax_weighted_sum(s, V[:, g, :])
    return out


def decode_sequence(q, k_cache, v_cache, block_tables, L, b, scale, softcap,
                    window, dtype):
    """float64 output [Hq, D] of sequence b (its one query is the newest
    token, so its context is all L positions)."""
    return attend(q[b], k_cache, v_cache, block_tables, b, L, scale, softcap,
                  window, dtype)


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, softcap=0.0,
           window=0, dtype="f32", seqs=None):
    """float64 output [B, Hq, D] (rows of sequences not in ``seqs`` are 0)."""
    B, Hq, D = q.shape
    if k_cache.shape[2] == 0 or Hq % k_cache.shape[2]:
        raise ValueError("num query heads must be a multiple of num kv heads")
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in (range(B) if seqs is None else seqs):
        out[b] = decode_sequence(q, k_cache, v_cache, block_tables,
                                 int(context_lens[b]), b, scale, softcap,
                                 window, dtype)
    return out


# --------------------------------------------------------------------------
# multi-query attention (several new tokens per sequence)
# --------------------------------------------------------------------------
def query_positions(L: int, n: int) -> np.ndarray:
    """Positions of a sequence's n new query tokens: the last n of its L
    (context_lens counts every new token, as it counts the one new token of
    a decode step)."""
    return np.arange(L - n, L)


def multi_query(q, query_start, k_cache, v_cache, block_tables, context_lens, scale,
                softcap=0.0, window=0, dtype="f32"):
    """float64 output [T, Hq, D] for T query tokens packed sequence by
    sequence: rows query_start[b] .. query_start[b+1]-1 are sequence b's new
    tokens in position order.  A token at position pos is causal: it sees
    the keys at positions up to and including its own, i.e. it is the decode
    query of a context of pos + 1 tokens (the window counts back from pos)."""
    T, Hq, D = q.shape
    if k_cache.shape[2] == 0 or Hq % k_cache.shape[2]:
        raise ValueError("num query heads must be a multiple of num kv heads")
    qs = np.asarray(query_start, dtype=np.int64)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for b in range(len(qs) - 1):
        n = int(qs[b + 1] - qs[b])
        L = int(context_lens[b])
        if n > L:
            raise ValueError("a sequence has more new tokens than context")
        for i, pos in enumerate(query_positions(L, n)):
            out[qs[b] + i] = attend(q[qs[b] + i], k_cache, v_cache, block_tables, b,
                                    int(pos) + 1, scale, softcap, window, dtype)
    return out


def multi_query_case(case):
    """Run the step a multi-query case describes: every new token's K/V row
    lands first, then attention."""
    kc, vc = case.k_cache, case.v_cache
    if case.slot_mapping is not None:
        kc, vc = reshape_and_cache(case.key, case.value, kc, vc, case.slot_mapping)
    return multi_query(case.q, case.query_start, kc, vc, case.block_tables,
                       case.context_lens, case.scale, case.softcap, case.window, case.dtype)


def decode_case(case, seqs=None):
    """Run the step a case describes: the new rows land first, then decode."""
    kc, vc = case.k_cache, case.v_cache
    if case.slot_mapping is not None:
        kc, vc = reshape_and_cache(case.key, case.value, kc, vc, case.slot_mapping)
    return decode(case.q, kc, vc, case.block_tables, case.context_lens,
                  case.scale, case.softcap, case.window, case.dtype, seqs=seqs)
