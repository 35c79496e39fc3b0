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
  if (w == 0) {
    // wavefront 0 scans the (at most 16) wavefront sums
    const int nw = (int)(blockDim.x >> 6);
    const int y = lane < nw ? s_tmp[lane] : 0;
    int z = y;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int u = __shfl_up(z, d, 64);
      if (lane >= d) z += u;
    }
    if (lane < nw) s_tmp[lane] = z - y;
    if (lane == nw - 1) s_tmp[16] = z;
  }
  __syncthreads();
  const int r = x - v + s_tmp[w];
  *total = s_tmp[16];
  __syncthreads();
  return r;
}

// Exclusive prefix sum of h[0, 256) in place by one wavefront (4 entries a
// lane); returns the sum.  The caller brackets it with workgroup barriers.
__device__ __forceinline__ int wave_scan_256(int* h) {
  const int lane = threadIdx.x & 63;
  const int a = h[4 * lane], b = h[4 * lane + 1], c = h[4 * lane + 2], d = h[4 * lane + 3];
  const int own = a + b + c + d;
  int z = own;
#pragma unroll
  for (int k = 1; k < 64; k <<= 1) {
    const int u = __shfl_up(z, k, 64);
    if (lane >= k) z += u;
  }
  const int base = z - own;
  h[4 * lane] = base;
  h[4 * lane + 1] = base + a;
  h[4 * lane + 2] = base + a + b;
  h[4 * lane + 3] = base + a + b + c;
  return __shfl(z, 63, 64);
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
  // (float scaling: only the order matters, and it is monotonic)
  const float inv_span = (float)(NBK - 1) / (float)span;
  auto bucket = [&](int L) {
    const int n = window > 0 ? min(L, window) : L;
    return NBK - 1 - min(NBK - 1, (int)((float)n * inv_span));
  };
  for (int b = t; b < num_seqs; b += blockDim.x) atomicAdd(&hist[bucket(length(b))], 1);
  __syncthreads();
  if (t < 64) wave_scan_256(hist);
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

// Rows 4 wg .. 4 wg + 3 of a step's new K/V rows, 256 threads a row.
__device__ __forceinline__ void copy_new_rows(const uint4* key, const uint4* value,
                                              uint4* k_cache, uint4* v_cache,
                                              const int64_t* slot_mapping, int num_tokens,
                                              int64_t num_slots, int row16, int wg) {
  const int i = wg * 4 + (int)(threadIdx.x >> 8);
  if (i >= num_tokens) return;
  const int64_t s = slot_mapping[i];
  if (s < 0 || s >= num_slots) return;
  const uint4* ks = key + (int64_t)i * row16;
  const uint4* vs = value + (int64_t)i * row16;
  uint4* kd = k_cache + s * row16;
  uint4* vd = v_cache + s * row16;
  for (int j = threadIdx.x & 255; j < row16; j += 256) {
    kd[j] = ks[j];
    vd[j] = vs[j];
  }
}

__global__ __launch_bounds__(1024) void step_prep_kernel(PrepParams pp) {
  if (blockIdx.x == 0) {
    if (pp.plan.order != nullptr)
      plan_body(pp.context_lens, pp.num_seqs, pp.max_context_len, pp.window, pp.part, pp.plan);
    return;
  }
  copy_new_rows(pp.key, pp.value, pp.k_cache, pp.v_cache, pp.slot_mapping, pp.num_tokens,
                pp.num_slots, pp.row16, (int)blockIdx.x - 1);
}

// A multi-query step's new K/V rows (the copy of reshape_cache_kernel).
struct NewRows {
  const uint4* key;      // [num_tokens, row16]
  const uint4* value;
  uint4* k_cache;        // [num_slots, row16]
  uint4* v_cache;
  const int64_t* slot_mapping;
  int num_tokens;
  int64_t num_slots;
  int row16;
};

// Arguments of the multi-query plan (described below).
struct MQPlanArgs {
  const int32_t* query_start;
  const int32_t* context_lens;
  int num_seqs, num_tokens, max_context_len, window, G, R;
  int2* tiles;
  int tile_cap;
  int32_t* num_tiles;
  int part_size;
  int2* units;
  int unit_cap;
  int32_t* vctx;
  int32_t* vrow;
};

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
//   atomics' (a tile's results do not depend on it).
//   units = (tile, partition) for every partition of part_size keys that a
//   tile's key span meets (keys split), sorted the same way by their work
//   (the keys the pair covers times the wavefronts, of the four R / 4-row
//   ones, that hold rows of the tile), and their count in num_tiles[1].  A
//   launch over this list holds no empty units, and consecutive workgroups
//   carry similar work: the dispatcher deals them to the shader engines of
//   an XCD in turn (stalling when the next one is full) and to an engine's
//   CUs in turn, so each run of 256 workgroups puts one on every CU and the
//   heaviest units spread evenly.
//   Null outputs are skipped (vctx and vrow together skip the token loop).
__device__ __forceinline__ void mq_plan_body(const MQPlanArgs& a) {
  const int32_t* __restrict__ query_start = a.query_start;
  const int32_t* __restrict__ context_lens = a.context_lens;
  const int num_seqs = a.num_seqs, num_tokens = a.num_tokens;
  const int max_context_len = a.max_context_len, window = a.window, G = a.G, R = a.R;
  int2* tiles = a.tiles;
  const int tile_cap = a.tile_cap;
  int32_t* num_tiles = a.num_tiles;
  const int part_size = a.part_size;
  int2* units = a.units;
  const int unit_cap = a.unit_cap;
  int32_t* vctx = a.vctx;
  int32_t* vrow = a.vrow;
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
  __shared__ int uhist[NBK];
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
    const int P = part_size;
    // the keys a tile's rows attend to: [klo, khi)
    auto keys_of = [&](int n, int L, int f0, int& klo, int& khi) {
      const int p_first = L - n + f0 / G;
      khi = L - n + (min(f0 + R, n * G) - 1) / G + 1;
      klo = window > 0 ? max(0, p_first + 1 - window) : 0;
    };
    // 256 levels of work, the most in bucket 0 (float scaling: only the
    // order matters, and it is monotonic)
    const float inv_span = (float)(NBK - 1) / (float)span;
    // a unit's work: keys x wavefronts holding rows (of four, R / 4 rows each)
    const float inv_part = P > 0 ? (float)(NBK - 1) / (float)(4 * P) : 0.0f;
    const int rw = max(R >> 2, 1);
    auto bucket = [&](int work, float inv) {
      return NBK - 1 - min(NBK - 1, (int)((float)max(work, 0) * inv));
    };
    // a tile's units: the partitions [pf, pl] its keys meet, bucketed by
    // their work; f(part, count, bucket) takes `count` partitions from `part`
    // on (the whole ones between the first and the last, P keys each, in one
    // call)
    auto for_units = [&](int klo, int khi, int rows, auto&& f) {
      if (khi <= klo) return;
      const int w = min((rows + rw - 1) / rw, 4);
      const int pf = klo / P;
      const int pl = (khi - 1) / P;
      if (pf == pl) {
        f(pf, 1, bucket((khi - klo) * w, inv_part));
        return;
      }
      f(pf, 1, bucket((pf * P + P - klo) * w, inv_part));
      if (pl - pf > 1) f(pf + 1, pl - pf - 1, bucket(P * w, inv_part));
      f(pl, 1, bucket((khi - pl * P) * w, inv_part));
    };
    if (t < NBK) hist[t] = 0;
    if (t < NBK) uhist[t] = 0;
    __syncthreads();
    // (up to 1024 sequences the second pass reuses the first's lists)
    const bool one = num_seqs <= (int)blockDim.x;
    int count = 0, total = 0, nu = 0;
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
          int klo, khi;
          keys_of(s_n[kk], s_L[kk], f0, klo, khi);
          const int bk = bucket(khi - klo, inv_span);
          const int rows = min(R, s_n[kk] * G - f0);
          if (pass == 0) {
            atomicAdd(&hist[bk], 1);
            if (units != nullptr)
              for_units(klo, khi, rows, [&](int, int c, int ub) { atomicAdd(&uhist[ub], c); });
          } else {
            const int idx = atomicAdd(&hist[bk], 1);
            if (idx < tile_cap) {
              tiles[idx] = make_int2(s_seq[kk], f0);
              if (units != nullptr)
                for_units(klo, khi, rows, [&](int part, int c, int ub) {
                  const int u = atomicAdd(&uhist[ub], c);
                  for (int k = 0; k < c && u + k < unit_cap; ++k)
                    units[u + k] = make_int2(idx, part + k);
                });
            }
          }
        });
        if (pass == 0) count += total;
        __syncthreads();
      }
      if (pass == 0) {
        // bucket offsets: wavefront 0 scans the tiles', wavefront 1 the units'
        if (t < 64) wave_scan_256(hist);
        else if (t < 128 && units != nullptr) {
          const int all = wave_scan_256(uhist);
          if (t == 64) s_tmp[16] = all;
        }
        __syncthreads();
        if (units != nullptr) nu = s_tmp[16];
      }
    }
    if (t == 0) *num_tiles = min(count, tile_cap);
    if (t == 0 && units != nullptr) num_tiles[1] = min(nu, unit_cap);
  }
  if (vctx == nullptr && vrow == nullptr) return;
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
    if (vctx != nullptr) vctx[tok] = min(max(pos + 1, 0), max_context_len);
    if (vrow != nullptr) vrow[tok] = lo;
  }
}

__global__ __launch_bounds__(1024) void mq_plan_kernel(MQPlanArgs a) { mq_plan_body(a); }

// A multi-query step's one launch before the attention: workgroup 0 builds
// the plan, workgroups 1.. copy the new K/V rows, every thread moving 16
// bytes of K and of V per step over all rows' 16-byte pieces (a prompt's
// rows can be short and many: 8,192 of 512 bytes).
__global__ __launch_bounds__(1024) void mq_step_prep_kernel(MQPlanArgs a, NewRows r) {
  if (blockIdx.x == 0) {
    mq_plan_body(a);
    return;
  }
  const int64_t n = (int64_t)r.num_tokens * r.row16;
  const int64_t stride = (int64_t)(gridDim.x - 1) * blockDim.x;
  for (int64_t e = (int64_t)(blockIdx.x - 1) * blockDim.x + threadIdx.x; e < n; e += stride) {
    const int i = (int)(e / r.row16);
    const int j = (int)(e - (int64_t)i * r.row16);
    const int64_t s = r.slot_mapping[i];
    if (s < 0 || s >= r.num_slots) continue;
    r.k_cache[s * r.row16 + j] = r.key[e];
    r.v_cache[s * r.row16 + j] = r.value[e];
  }
}

}  // namespace pa
