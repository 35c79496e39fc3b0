// Work plan for pa_decode: one workgroup sorts the sequences by attended
// length, longest first, and (for launches that loop over work) lists every
// (sequence, partition) that holds keys, so no workgroup is spent on
// partitions past a sequence's end.
#pragma once

#include "pa_device.h"

namespace pa {

struct Plan {
  int32_t* order;      // [B] sequences, longest first
  int32_t* num_items;  // [1] number of items
  int2* items;         // [<= B * NP] (sequence, partition); null: not listed
};

// Exclusive prefix sum over the workgroup; *total gets the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_tmp[w] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int k = 0; k < (int)(blockDim.x >> 6); ++k) {
      const int t = s_tmp[k];
      s_tmp[k] = run;
      run += t;
    }
    s_tmp[16] = run;
  }
  __syncthreads();
  const int r = x - v + s_tmp[w];
  *total = s_tmp[16];
  __syncthreads();
  return r;
}

// Expands nk lists into one array of `total` entries, all threads writing:
// list k starts at s_off[k] (exclusive offsets, non-decreasing) and ends
// where the next list starts, so entry idx belongs to the last k with
// s_off[k] <= idx.  emit(k, i, idx) writes entry i of list k at idx.
template <typename Emit>
__device__ __forceinline__ void expand_lists(const int* s_off, int nk, int total, Emit&& emit) {
  for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
    int lo = 0, hi = nk - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[mid] <= idx) lo = mid;
      else hi = mid - 1;
    }
    emit(lo, idx - s_off[lo], idx);
  }
}

// The plan, built by one workgroup of 1024 threads.  part: partition size
// in tokens (max_context_len when keys are not split).
__device__ __forceinline__ void plan_body(const int32_t* __restrict__ context_lens, int num_seqs,
                                          int max_context_len, int window, int part,
                                          const Plan& plan) {
  constexpr int NBK = 256;
  __shared__ int hist[NBK];
  __shared__ int s_tmp[17];
  __shared__ int s_off[1024];
  __shared__ int s_seq[1024];
  __shared__ int s_first[1024];
  const int t = threadIdx.x;
  if (t < NBK) hist[t] = 0;
  __syncthreads();
  const int span = max(max_context_len, 1);
  auto length = [&](int b) { return min(max(context_lens[b], 0), max_context_len); };
  // counting sort over 256 length buckets, descending: the longest
  // sequences land in bucket 0 (order within a bucket is arbitrary, which
  // no result depends on)
  auto bucket = [&](int L) {
    const int n = window > 0 ? min(L, window) : L;
    return NBK - 1 - (int)(((long long)n * (NBK - 1)) / span);
  };
  for (int b = t; b < num_seqs; b += blockDim.x) atomicAdd(&hist[bucket(length(b))], 1);
  __syncthreads();
  {
    int total;
    const int off = block_exclusive_scan(t < NBK ? hist[t] : 0, s_tmp, &total);
    if (t < NBK) hist[t] = off;
  }
  __syncthreads();
  for (int b = t; b < num_seqs; b += blockDim.x)
    plan.order[atomicAdd(&hist[bucket(length(b))], 1)] = b;
  if (plan.items == nullptr) return;
  __syncthreads();

  // the non-empty partitions of each sequence, sequences in plan order; an
  // empty sequence keeps one item (its partition 0 writes the zero output)
  int base = 0;
  for (int k0 = 0; k0 < num_seqs; k0 += blockDim.x) {
    const int k = k0 + t;
    int b = 0, first = 0, n = 0;
    if (k < num_seqs) {
      b = plan.order[k];
      const int L = length(b);
      if (L <= 0) {
        n = 1;
      } else {
        const int start = window > 0 ? max(0, L - window) : 0;
        first = start / part;
        n = (L - 1) / part - first + 1;
      }
    }
    int total;
    s_off[t] = block_exclusive_scan(n, s_tmp, &total);
    s_seq[t] = b;
    s_first[t] = first;
    __syncthreads();
    int2* items = plan.items + base;
    expand_lists(s_off, blockDim.x, total, [&](int kk, int i, int idx) {
      items[idx] = make_int2(s_seq[kk], s_first[kk] + i);
    });
    base += total;
    __syncthreads();
  }
  if (t == 0) *plan.num_items = base;
}

__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ context_lens,
                                                    int num_seqs, int max_context_len, int window,
                                                    int part, Plan plan) {
  plan_body(context_lens, num_seqs, max_context_len, window, part, plan);
}

// What a layer step does before its decode launch, in one launch of
// 1024-thread workgroups: workgroup 0 builds the plan (when plan.order is
// set); workgroups 1.. copy the new K/V rows into their slots, four tokens
// per workgroup (the copy of reshape_cache_kernel: 16-byte moves, slots
// outside the cache skipped).
struct PrepParams {
  const int32_t* context_lens;
  int num_seqs, max_context_len, window, part;
  Plan plan;             // order null: no plan
  const uint4* key;      // [num_tokens, row16]
  const uint4* value;
  uint4* k_cache;        // [num_slots, row16]
  uint4* v_cache;
  const int64_t* slot_mapping;
  int num_tokens;
  int64_t num_slots;
  int row16;
};

__global__ __launch_bounds__(1024) void step_prep_kernel(PrepParams pp) {
  if (blockIdx.x == 0) {
    if (pp.plan.order != nullptr)
      plan_body(pp.context_lens, pp.num_seqs, pp.max_context_len, pp.window, pp.part, pp.plan);
    return;
  }
  const int i = (int)(blockIdx.x - 1) * 4 + (int)(threadIdx.x >> 8);
  if (i >= pp.num_tokens) return;
  const int64_t s = pp.slot_mapping[i];
  if (s < 0 || s >= pp.num_slots) return;
  const uint4* ks = pp.key + (int64_t)i * pp.row16;
  const uint4* vs = pp.value + (int64_t)i * pp.row16;
  uint4* kd = pp.k_cache + s * pp.row16;
  uint4* vd = pp.v_cache + s * pp.row16;
  for (int j = threadIdx.x & 255; j < pp.row16; j += 256) {
    kd[j] = ks[j];
    vd[j] = vs[j];
  }
}

// Plan of a multi-query launch (one workgroup of 1024 threads):
//   vctx[tok] = context of query token tok (its position + 1, clamped to
//   [0, max_context_len]); vrow[tok] = its sequence (per-token path);
//   tiles = (sequence, first row) for every R rows of each sequence's
//   n * G rows (tiled path), at most tile_cap of them, the most work first
//   over all sequences: a tile's work is the span of keys its rows attend
//   to (from its first row's window start to its last row's position),
//   bucketed into 256 levels, and a counting sort (count, then place) puts
//   the tiles in bucket order, so the grid dispatches the longest tiles of
//   every sequence before any short one.  Within a bucket the order is the
//   atomics' (a tile's results do not depend on it).  Null outputs are
//   skipped.
__global__ __launch_bounds__(1024) void mq_plan_kernel(const int32_t* __restrict__ query_start,
                                                       const int32_t* __restrict__ context_lens,
                                                       int num_seqs, int num_tokens,
                                                       int max_context_len, int window, int G,
                                                       int R, int2* tiles, int tile_cap,
                                                       int32_t* num_tiles, int32_t* vctx,
                                                       int32_t* vrow) {
  constexpr int kQS = 4096;  // sequence starts and contexts kept in LDS up to this many
  constexpr int NBK = 256;
  __shared__ int s_tmp[17];
  __shared__ int s_off[1024];
  __shared__ int s_nt[1024];
  __shared__ int s_seq[1024];
  __shared__ int s_n[1024];
  __shared__ int s_L[1024];
  __shared__ int s_qs[kQS + 1];
  __shared__ int s_cl[kQS];
  __shared__ int hist[NBK];
  const int t = threadIdx.x;
  const bool in_lds = num_seqs <= kQS;
  if (in_lds) {
    for (int b = t; b <= num_seqs; b += blockDim.x) s_qs[b] = query_start[b];
    for (int b = t; b < num_seqs; b += blockDim.x) s_cl[b] = context_lens[b];
  }
  __syncthreads();
  auto qstart = [&](int b) { return in_lds ? s_qs[b] : query_start[b]; };
  auto ctx = [&](int b) { return in_lds ? s_cl[b] : context_lens[b]; };
  if (tiles != nullptr) {
    const int span = max(max_context_len, 1);
    auto bucket = [&](int n, int L, int f0) {
      const int p_first = L - n + f0 / G;
      const int p_last = L - n + (min(f0 + R, n * G) - 1) / G;
      const int klo = window > 0 ? max(0, p_first + 1 - window) : 0;
      const int work = min(max(p_last + 1 - klo, 0), span);
      return NBK - 1 - (int)(((long long)work * (NBK - 1)) / span);
    };
    if (t < NBK) hist[t] = 0;
    __syncthreads();
    // (up to 1024 sequences the second pass reuses the first's lists)
    const bool one = num_seqs <= (int)blockDim.x;
    int count = 0, total = 0;
    for (int pass = 0; pass < 2; ++pass) {
      for (int k0 = 0; k0 < num_seqs; k0 += blockDim.x) {
        if (pass == 0 || !one) {
          const int b = k0 + t;
          int nt = 0, n = 0, L = 0;
          if (b < num_seqs) {
            // rows of the sequence's tokens that lie in [0, num_tokens)
            const int q0 = min(max(qstart(b), 0), num_tokens);
            n = min(max(qstart(b + 1) - q0, 0), num_tokens - q0);
            nt = (n * G + R - 1) / R;
            L = min(ctx(b), max_context_len);
          }
          s_off[t] = block_exclusive_scan(nt, s_tmp, &total);
          s_nt[t] = nt;
          s_seq[t] = b;
          s_n[t] = n;
          s_L[t] = L;
          __syncthreads();
        }
        // a sequence's tiles from its last rows (the most keys) down
        const int nk = min(num_seqs - k0, (int)blockDim.x);
        expand_lists(s_off, nk, total, [&](int kk, int i, int) {
          const int f0 = (s_nt[kk] - 1 - i) * R;
          const int bk = bucket(s_n[kk], s_L[kk], f0);
          if (pass == 0) {
            atomicAdd(&hist[bk], 1);
          } else {
            const int idx = atomicAdd(&hist[bk], 1);
            if (idx < tile_cap) tiles[idx] = make_int2(s_seq[kk], f0);
          }
        });
        if (pass == 0) count += total;
        __syncthreads();
      }
      if (pass == 0) {
        int all;
        const int off = block_exclusive_scan(t < NBK ? hist[t] : 0, s_tmp, &all);
        if (t < NBK) hist[t] = off;
        __syncthreads();
      }
    }
    if (t == 0) *num_tiles = min(count, tile_cap);
  }
  for (int tok = t; tok < num_tokens; tok += blockDim.x) {
    // the sequence that owns tok: the last b with query_start[b] <= tok
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (qstart(mid) <= tok) lo = mid;
      else hi = mid - 1;
    }
    const int q0 = qstart(lo);
    const int n = qstart(lo + 1) - q0;
    const int pos = ctx(lo) - n + (tok - q0);
    vctx[tok] = min(max(pos + 1, 0), max_context_len);
    if (vrow != nullptr) vrow[tok] = lo;
  }
}

}  // namespace pa
