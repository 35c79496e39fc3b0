// gfx950 kernels for paged decode attention: the split-K decode pass, the
// partition reduce and the KV-cache scatter.
//
// Decode work unit: one workgroup per (sequence b, KV head g, partition p),
// with 1..8 wavefronts that take the partition's chunks round-robin and are
// merged in LDS at the end.  Within a wavefront:
//   * a K/V row of head g (D elements) is spread over LPR lanes, 16 bytes
//     per lane, so one load instruction fetches RPI = 64/LPR whole rows and a
//     chunk of NI instructions covers NT = RPI*NI tokens with coalesced 16-B
//     loads (a whole page when block_size == NT);
//   * the G query heads that share KV head g stay in registers as 16-byte
//     fragments matching the lane's slice of every row;
//   * q.k partial sums (NI rows x G heads per lane) are reduce-scattered
//     across the LPR lanes of a row, one useful value per shuffle;
//   * the chunk's logits go through LDS, where lane l owns query head l % G
//     for the online-softmax update (max and sum by xor shuffles), and the
//     resulting probabilities are read back as broadcasts for P.V;
//   * P.V accumulates into G x (elements per lane) float32 registers.
// Next-chunk K loads are issued as soon as the current K fragments are
// consumed and next-chunk V loads as soon as P.V is done, so each wavefront
// keeps a chunk of K and V in flight while it computes.
#pragma once

#include <type_traits>

#include "pa_device.h"

namespace pa {

constexpr int kMaxWaves = 8;

struct DecodeParams {
  void* out;               // [B, Hq, D]
  const int32_t* order;      // [B] sequences, longest first (workspace); null: 0, 1, ...
  const int32_t* num_items;  // looping launches: number of work items
  const int2* items;         // looping launches: (sequence, partition) list
  float* tmp_out;          // [B, Hq, NP, D]
  float* max_logits;       // [B, Hq, NP], base-2 logits
  float* exp_sums;         // [B, Hq, NP]
  const void* q;           // [B, Hq, D]
  const void* k_cache;     // [NB, bs, Hkv, D]
  const void* v_cache;
  const int32_t* block_tables;  // [B, max_blocks_per_seq]
  const int32_t* context_lens;  // [B]
  const int32_t* seq_row;  // null, or [B] block-table row of each unit sequence
  int max_blocks_per_seq;
  int max_context_len;
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int num_blocks;
  int log2_bs;
  int window;              // > 0: last `window` keys only
  int part;                // partition size in tokens (> 0)
  int num_parts;           // NP
  float qk_mul;            // multiplies q.k
  float cap_mul;           // > 0: logit2 = cap_mul * tanh(q.k * qk_mul)
  int xcd_units;           // > 0: XCD-grouped grid over this many (b, p) units
  int prio;                // chunks per wave-priority step (0: none)
  // Tail rows (vector kernel): row b of tail_k / tail_v [B, Hkv, D] is the
  // newest token of sequence b, to be written at slot tail_slots[b]; null:
  // the caches already hold every row
  const void* tail_k;
  const void* tail_v;
  const int64_t* tail_slots;
};

struct ReduceParams {
  void* out;
  const float* tmp_out;
  const float* max_logits;
  const float* exp_sums;
  const int32_t* context_lens;
  int max_context_len;
  int num_seqs;
  int num_heads;
  int window;
  int part;
  int num_parts;
};

template <int DT, int D, int G>
struct DecodeShape {
  static constexpr int EB = Elem<DT>::bytes;
  static constexpr int EPL = 16 / EB;                 // elements per lane per load
  static constexpr int LPR = D / EPL;                 // lanes per row
  static constexpr int RPI = 64 / LPR;                // rows per load instruction
  static constexpr int NI = (G >= 8) ? 4 : 8;         // load instructions per chunk
  static constexpr int NT = RPI * NI;                 // tokens per chunk
  static constexpr int NV = NI * G;                   // partial dots per lane
  static constexpr int R = NV >= LPR ? NV / LPR : 1;  // finished dots per lane
  static constexpr int SLOTS = NT * G;                // logits per chunk
  static constexpr int SPL = SLOTS >= 64 ? SLOTS / 64 : 1;
  // LDS floats per wavefront: logits, rescale, table window, max/sum, acc
  static constexpr int LDS_FLOATS = SLOTS + G + 64 + 2 * G + G * D;
  static_assert(LPR >= 2 && LPR <= 64, "row must span 2..64 lanes");
  static_assert((G & (G - 1)) == 0 && G <= 64, "group size must be a power of two");
};

// Block-table row of sequence b.  Multi-query launches run every query token
// as its own sequence (context = the keys up to the token's position), all
// of one sequence's tokens sharing its table row through seq_row.
__device__ __forceinline__ const int32_t* table_row(const DecodeParams& p, int b) {
  typedef const __attribute__((address_space(4))) int32_t cint32;
  const int row = p.seq_row ? ((cint32*)p.seq_row)[b] : b;
  return p.block_tables + (size_t)row * p.max_blocks_per_seq;
}

// The (sequence, KV head, partition) unit of a decode workgroup.
struct Unit {
  int b, g, part, lo, hi;
  int L;        // the sequence's context length (clamped)
  bool single;  // the sequence's attended keys fall in this one partition
};

// Fills the unit's key range.  Returns false when it has no keys to attend
// to; partition 0 of an empty sequence writes its zero output (by the whole
// workgroup, or with HEADS by the head's own wavefront).
template <int DT, int D, int G, bool HEADS = false>
__device__ __forceinline__ bool unit_range(const DecodeParams& p, Unit& u) {
  typedef const __attribute__((address_space(4))) int32_t cint32;
  const int L = min(((cint32*)p.context_lens)[u.b], p.max_context_len);
  if (L <= 0) {
    const int first = HEADS ? (int)(threadIdx.x & 63) : (int)threadIdx.x;
    const int stride = HEADS ? 64 : (int)blockDim.x;
    if (u.part == 0)
      for (int i = first; i < G * D; i += stride)
        store_elem<DT>(p.out, ((size_t)u.b * p.num_heads + (size_t)u.g * G) * D + i, 0.0f);
    return false;
  }
  const int P = p.part;
  const int start = p.window > 0 ? max(0, L - p.window) : 0;
  u.L = L;
  u.lo = max(start, u.part * P);
  u.hi = min(L, u.part * P + P);
  u.single = (start / P) == ((L - 1) / P);
  return u.lo < u.hi;
}

// One unit per workgroup: KV head fastest, then sequences in the plan's
// longest-first order, then partitions (so a sequence's partitions are
// spread over the whole dispatch).  HEADS: the workgroup holds every KV head
// of its (sequence, partition), wavefront w taking head w.
//
// XCD grouping (xcd_units > 0): workgroups are handed to the eight XCDs in
// turn (workgroup i to XCD i mod 8), so workgroup i is read as slot i / 8 of
// XCD i mod 8, and the KV heads of one (sequence, partition) take
// consecutive slots of the same XCD: a token's rows of all heads (adjacent
// in memory) are then fetched through one L2.  The grid is padded to a
// multiple of 8 * Hkv; padding workgroups have no unit.
template <int DT, int D, int G, bool HEADS = false>
__device__ __forceinline__ bool grid_unit(const DecodeParams& p, Unit& u) {
  typedef const __attribute__((address_space(4))) int32_t cint32;
  const int id = blockIdx.x;
  int rest;
  if (!HEADS && p.xcd_units > 0) {
    const int slot = id >> 3;
    u.g = slot % p.num_kv_heads;
    rest = (slot / p.num_kv_heads) * 8 + (id & 7);
    if (rest >= p.xcd_units) return false;
  } else {
    u.g = HEADS ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : id % p.num_kv_heads;
    rest = HEADS ? id : id / p.num_kv_heads;
  }
  u.part = rest / p.num_seqs;
  u.b = p.order ? ((cint32*)p.order)[rest % p.num_seqs] : rest % p.num_seqs;
  return unit_range<DT, D, G, HEADS>(p, u);
}

// Unit `it` of a looping launch: KV head fastest over the plan's item list
// (HEADS: item `it` for every head, head = wavefront).
template <int DT, int D, int G, bool HEADS = false>
__device__ __forceinline__ bool item_unit(const DecodeParams& p, int it, Unit& u) {
  typedef const __attribute__((address_space(4))) uint64_t cu64;
  u.g = HEADS ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : it % p.num_kv_heads;
  // an item is (sequence, partition) as two int32, little-endian
  const uint64_t item = ((cu64*)p.items)[HEADS ? it : it / p.num_kv_heads];
  u.b = (int)(uint32_t)item;
  u.part = (int)(uint32_t)(item >> 32);
  return unit_range<DT, D, G, HEADS>(p, u);
}

// Runs body(unit) for this workgroup's units: its own one, or (LOOP) every
// gridDim-th unit of the plan's list, so that a launch whose grid would be
// mostly empty partitions stays small.
template <int DT, int D, int G, bool LOOP, bool HEADS = false, typename Body>
__device__ __forceinline__ void for_units(const DecodeParams& p, Body&& body) {
  if constexpr (LOOP) {
    typedef const __attribute__((address_space(4))) int32_t cint32;
    const int n = *(cint32*)p.num_items * (HEADS ? 1 : p.num_kv_heads);
    for (int it = blockIdx.x; it < n; it += gridDim.x) {
      Unit u;
      if (item_unit<DT, D, G, HEADS>(p, it, u)) body(u);
      __syncthreads();  // LDS is reused by the next unit
    }
  } else {
    Unit u;
    if (grid_unit<DT, D, G, HEADS>(p, u)) body(u);
  }
}

// Merges the wavefronts' running (max, sum, accumulators) and writes the
// unit's G output rows, or its split-K partials.  Wavefront v's record
// starts at smem + v * stride: maxima at +ml, sums at +ml + G, accumulators
// [G][row_stride] at +acc.
template <int DT, int D, int G>
__device__ __forceinline__ void merge_store(const DecodeParams& p, const Unit& u,
                                            const float* smem, int stride, int ml, int acc,
                                            int nw, int row_stride = D) {
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
    const int h = i / D;
    const int d = i % D;
    float M = kNegInf;
    for (int v = 0; v < nw; ++v) M = fmaxf(M, smem[v * stride + ml + h]);
    float den = 0.0f, num = 0.0f;
    for (int v = 0; v < nw; ++v) {
      const float* lv = smem + v * stride;
      const float f = fast_exp2(lv[ml + h] - M);
      den += f * lv[ml + G + h];
      num += f * lv[acc + h * row_stride + d];
    }
    const size_t hq = (size_t)u.g * G + h;
    if (u.single) {
      store_elem<DT>(p.out, ((size_t)u.b * p.num_heads + hq) * D + d, num / den);
    } else {
      const size_t pi = ((size_t)u.b * p.num_heads + hq) * p.num_parts + u.part;
      p.tmp_out[pi * D + d] = num / den;
      if (d == 0) {
        p.max_logits[pi] = M;
        p.exp_sums[pi] = den;
      }
    }
  }
}

// PAGED: every chunk lies inside one KV page (block_size >= NT), so a
// chunk's rows share one physical block: its base address is wave-uniform
// (scalar registers) and each lane adds a 32-bit row offset.  Otherwise each
// row looks up its own block.
#ifndef PA_DECODE_MIN_WAVES
#define PA_DECODE_MIN_WAVES 1
#endif
// TAIL: the launch writes the new tail rows itself (p.tail_slots set).
template <int DT, int D, int G, bool PAGED, bool LOOP, bool TAIL = false>
__global__ __launch_bounds__(64 * kMaxWaves, PA_DECODE_MIN_WAVES) void decode_kernel(DecodeParams p) {
  using S = DecodeShape<DT, D, G>;
  constexpr int EB = S::EB, EPL = S::EPL, LPR = S::LPR, RPI = S::RPI;
  constexpr int NI = S::NI, NT = S::NT, NV = S::NV, R = S::R;
  constexpr int SLOTS = S::SLOTS, SPL = S::SPL;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  // The parameters a unit's first loads depend on, all read here at once:
  // left to the compiler, they came in three dependent rounds of kernel
  // argument loads, each behind a branch, before the sequence's length
  // could be requested.
  asm volatile("" ::"s"(p.order), "s"(p.context_lens), "s"(p.block_tables), "s"(p.q),
               "s"(p.k_cache), "s"(p.v_cache), "s"(p.seq_row), "s"(p.num_seqs),
               "s"(p.num_kv_heads), "s"(p.max_context_len), "s"(p.max_blocks_per_seq),
               "s"(p.window), "s"(p.part), "s"(p.xcd_units), "s"(p.log2_bs), "s"(p.num_blocks),
               "s"(p.num_heads), "s"(p.prio), "s"(p.tail_k), "s"(p.tail_v), "s"(p.tail_slots),
               "s"(nw));

  // per-wavefront LDS, sized by the launch (decode_lds_bytes)
  extern __shared__ __align__(16) float smem[];
  float* s_wave = smem + w * S::LDS_FLOATS;
  float* sc = s_wave;                              // [SLOTS] logits / probabilities
  float* s_alpha = sc + SLOTS;                     // [G] rescale of this chunk
  int32_t* tbl = reinterpret_cast<int32_t*>(s_alpha + G);  // [64] block-table window
  float* s_ml = s_alpha + G + 64;                  // [2G] final max and sum
  float* s_acc = s_ml + 2 * G;                     // [G*D] final accumulators
  for_units<DT, D, G, LOOP>(p, [&](const Unit& u) {
  const int Hkv = p.num_kv_heads;
  const int Hq = p.num_heads;
  const int b = u.b, g = u.g, lo = u.lo, hi = u.hi;

  const int e0 = (lane % LPR) * EPL;  // first element of this lane's fragment
  const int rsub = lane / LPR;        // row of this lane within a load

  // query fragments of the G heads that read KV head g
  uint4 qf[G];
  {
    const char* qb = static_cast<const char*>(p.q) +
                     (((size_t)b * Hq + (size_t)g * G) * D + e0) * EB;
#pragma unroll
    for (int h = 0; h < G; ++h) qf[h] = ld16(qb + (size_t)h * D * EB);
  }

  // A window of 64 consecutive block-table entries per wavefront, in LDS.
  // Refilled (rarely: every 64 pages) inside a uniform branch, so the wait
  // for the refill never holds back the K/V loads already in flight.
  const int32_t* bt = table_row(p, b);
  const int log2_bs = p.log2_bs;
  const int last_pg = (hi - 1) >> log2_bs;
  int pg0 = -(1 << 30);
  auto refill = [&](int first) {
    pg0 = first;
    const int pg = first + lane;
    const int v = pg <= last_pg ? bt[pg] : 0;
    tbl[lane] = v;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  const uint32_t row_bytes = (uint32_t)(Hkv * D * EB);          // bytes between slots
  const uint32_t lane_bytes = (uint32_t)((g * D + e0) * EB);
  const uint32_t page_bytes = row_bytes << log2_bs;
  const char* kbase = static_cast<const char*>(p.k_cache);
  const char* vbase = static_cast<const char*>(p.v_cache);
  // harmless L2-resident target for the prefetch slot of the last chunk
  const char* dummy = static_cast<const char*>(p.q) + ((size_t)b * Hq + (size_t)g * G) * D * EB;
  const uint32_t dummy_off = (uint32_t)(e0 * EB);

  // Chunk c covers positions [c*NT, c*NT + NT).  Rows outside [lo, hi) are
  // clamped into it (their logits are masked later), so no unreferenced slot
  // (free block, page tail, table padding) is ever read.
  //   PAGED: one buffer descriptor per page (scalar registers), the chunk's
  //          offset in the page as the scalar offset, 32-bit row offsets;
  //   else:  per-row slot index (block * bs + offset), 64-bit addresses.
  struct Addr {
    rsrc_t kr, vr;
    uint32_t soff;
    uint32_t off[NI];
  };
  auto page_addr = [&](int c, int phys, Addr& a) {
    const int cs = c * NT;
    phys = ((unsigned)phys < (unsigned)p.num_blocks) ? phys : 0;
    const uint64_t base = (uint64_t)phys * page_bytes;
    a.kr = make_rsrc(kbase + base, page_bytes);
    a.vr = make_rsrc(vbase + base, page_bytes);
    a.soff = (uint32_t)(cs & ((1 << log2_bs) - 1)) * row_bytes;
    const int rlo = lo - cs, rhi = hi - 1 - cs;  // uniform clamp bounds
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = min(max(i * RPI + rsub, rlo), rhi);
      a.off[i] = (uint32_t)r * row_bytes + lane_bytes;
    }
  };
  auto chunk_addr = [&](int c, Addr& a) {
    const int cs = c * NT;
    const int cpg_lo = max(cs, lo) >> log2_bs;
    const int cpg_hi = (min(cs + NT, hi) - 1) >> log2_bs;
    if (cpg_lo < pg0 || cpg_hi - pg0 >= 64) refill(cpg_lo);
    if constexpr (PAGED) {
      page_addr(c, __builtin_amdgcn_readfirstlane(tbl[cpg_lo - pg0]), a);
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int pos = min(max(cs + i * RPI + rsub, lo), hi - 1);
        int phys = tbl[(pos >> log2_bs) - pg0];
        phys = ((unsigned)phys < (unsigned)p.num_blocks) ? phys : 0;
        a.off[i] = ((uint32_t)phys << log2_bs) | (uint32_t)(pos & ((1 << log2_bs) - 1));
      }
    }
  };
  auto kload = [&](const Addr& a, int i) -> uint4 {
    if constexpr (PAGED) return ld16_buf(a.kr, a.off[i], a.soff);
    else return ld16_stream(kbase + (uint64_t)a.off[i] * row_bytes + lane_bytes);
  };
  auto vload = [&](const Addr& a, int i) -> uint4 {
    if constexpr (PAGED) return ld16_buf(a.vr, a.off[i], a.soff);
    else return ld16_stream(vbase + (uint64_t)a.off[i] * row_bytes + lane_bytes);
  };
  auto dummy_addr = [&](Addr& a) {
    if constexpr (PAGED) {
      a.kr = make_rsrc(dummy, (uint32_t)(G * D * EB));
      a.vr = a.kr;
      a.soff = 0;
#pragma unroll
      for (int i = 0; i < NI; ++i) a.off[i] = dummy_off;
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) a.off[i] = 0;
    }
  };

  float m_run = kNegInf;  // running max (base 2) of query head lane % G
  float l_run = 0.0f;     // this lane's share of that head's running sum
  float acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.0f;

  uint4 kr[NI], vr[NI];
  Addr ad;

  const int c0 = lo / NT;
  const int c1 = (hi - 1) / NT;
  int c = c0 + w;
  if (c <= c1) {
    if constexpr (PAGED) {
      // first chunk: its block id through the scalar cache, so K/V loads
      // start before the block-table window arrives
      typedef const __attribute__((address_space(4))) int32_t cint32;
      const int cpg = max(c * NT, lo) >> log2_bs;
      page_addr(c, ((cint32*)bt)[cpg], ad);
      pg0 = cpg;
      const int v = cpg + lane <= last_pg ? bt[cpg + lane] : 0;
#pragma unroll
      for (int i = 0; i < NI; ++i) kr[i] = kload(ad, i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NI; ++i) vr[i] = vload(ad, i);
      __builtin_amdgcn_sched_barrier(0);
      tbl[lane] = v;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
      chunk_addr(c, ad);
      // issue all of K before any of V, as the loop does: the wait counter
      // then lets q.k start while V is still in flight
#pragma unroll
      for (int i = 0; i < NI; ++i) kr[i] = kload(ad, i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NI; ++i) vr[i] = vload(ad, i);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Tail rows (looked up after the first chunk's loads are in flight): the
  // unit holding the sequence's newest key (position L - 1) takes that
  // key's K/V from the new-row arrays, writes this head's slice of it to
  // its slot (wavefront 0, after its last chunk), and, when the slot is the
  // one the block table gives position L - 1, uses the new values wherever
  // it would read that slot (the key itself and the rows clamped onto it) --
  // the order reshape_and_cache-then-decode would give, with no launch in
  // between.
  bool tail = false, tail_store = false;
  int64_t slot = -1;
  uint4 k_tail = make_uint4(0, 0, 0, 0), v_tail = k_tail;
  if (TAIL && u.hi == u.L) {
    typedef const __attribute__((address_space(4))) int32_t cint32;
    typedef const __attribute__((address_space(4))) int64_t cint64;
    slot = ((cint64*)p.tail_slots)[b];
    if (slot >= 0 && slot < ((int64_t)p.num_blocks << log2_bs)) {
      const size_t src = ((size_t)b * Hkv * D + (size_t)g * D + e0) * EB;
      k_tail = ld16(static_cast<const char*>(p.tail_k) + src);
      v_tail = ld16(static_cast<const char*>(p.tail_v) + src);
      tail_store = true;
      const int last = u.L - 1;
      const int phys = ((cint32*)bt)[last >> log2_bs];
      tail = (unsigned)phys < (unsigned)p.num_blocks &&
             slot == ((int64_t)phys << log2_bs) + (last & ((1 << log2_bs) - 1));
    }
  }
  // the chunk holding position L - 1, and a row of it that reads that
  // position: row r's position c_tail * NT + r is clamped into [lo, L - 1]
  const int c_tail = tail ? (u.L - 1) / NT : -1;
  auto reads_tail = [&](int i) { return max(c_tail * NT + i * RPI + rsub, lo) >= u.L - 1; };
  // The tail row's loads were issued after the first chunk's: wait for
  // them here, once.  Left pending into the loop, they made the compiler's
  // wait before each chunk's q.k count from them, i.e. wait for every load
  // in flight, V of the chunk included, so that each chunk paid V's whole
  // round trip; the first chunk's K and V were issued together, so this
  // costs little.
  if constexpr (TAIL) __builtin_amdgcn_s_waitcnt(vmcnt_only(0));

#pragma clang loop unroll(disable)
  for (; c <= c1; c += nw) {
    // issue priority from the chunks this wavefront has left, in steps of
    // p.prio chunks (workgroups sharing a CU then finish together rather
    // than oldest first)
    if (p.prio) {
      const int rem = (c1 - c) / nw;
      if (rem >= 4 * p.prio) __builtin_amdgcn_s_setprio(3);
      else if (rem >= 2 * p.prio) __builtin_amdgcn_s_setprio(2);
      else if (rem >= p.prio) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
    if (TAIL && c == c_tail) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
        if (reads_tail(i)) kr[i] = k_tail;
    }
    // q.k partial sums over this lane's slice of each row
    float dots[NV];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int h = 0; h < G; ++h) dots[i * G + h] = dot16<DT>(kr[i], qf[h], 0.0f);

    // the next chunk's K goes in flight (the last chunk re-reads a few
    // L2-resident bytes instead, so the loads stay unconditional)
    __builtin_amdgcn_sched_barrier(0);
    if (c + nw <= c1) chunk_addr(c + nw, ad);
    else dummy_addr(ad);
#pragma unroll
    for (int i = 0; i < NI; ++i) kr[i] = kload(ad, i);
    __builtin_amdgcn_sched_barrier(0);

    TransposeReduce<NV, LPR / 2, NV>::run(dots, lane);
    const int jb = tr_base<NV, LPR>(lane);
    const int cs = c * NT;
    if (p.cap_mul > 0.0f) {
#pragma unroll
      for (int t = 0; t < R; ++t) dots[t] = p.cap_mul * tanh_def(dots[t] * p.qk_mul);
    } else {
#pragma unroll
      for (int t = 0; t < R; ++t) dots[t] *= p.qk_mul;
    }
#pragma unroll
    for (int t = 0; t < R; ++t) {
      const int j = jb + t;
      const int row = (j / G) * RPI + rsub;
      const int h = j % G;
      const int pos = cs + row;
      sc[row * G + h] = (pos >= lo && pos < hi) ? dots[t] : kNegInf;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // online softmax: lane owns query head lane % G
    float sv[SPL];
    float cmax = kNegInf;
#pragma unroll
    for (int k = 0; k < SPL; ++k) {
      const int idx = lane + 64 * k;
      sv[k] = idx < SLOTS ? sc[idx] : kNegInf;
      cmax = fmaxf(cmax, sv[k]);
    }
#pragma unroll
    for (int m = G; m < 64; m <<= 1) cmax = fmaxf(cmax, shfl_xor_f(cmax, m));
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = fast_exp2(m_run - m_new);
    float psum = 0.0f;
#pragma unroll
    for (int k = 0; k < SPL; ++k) {
      const int idx = lane + 64 * k;
      // 16-bit storage: the probability as P.V uses it (rounded to the
      // storage type), so the sum and the products see the same value
      const float pk = round_to<DT>(fast_exp2(sv[k] - m_new));
      psum += pk;
      if (idx < SLOTS) sc[idx] = pk;
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (lane < G) s_alpha[lane] = alpha;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // P.V
    if (TAIL && c == c_tail) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
        if (reads_tail(i)) vr[i] = v_tail;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float a = s_alpha[h];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= a;
    }
    if constexpr (DT == DT_F32) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float pr[G];
#pragma unroll
        for (int h = 0; h < G; ++h) pr[h] = sc[(i * RPI + rsub) * G + h];
        float ve[EPL];
        widen16<DT>(vr[i], ve);
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pr[h], ve[e], acc[h][e]);
      }
    } else {
      // 16-bit storage: loads i and i + 1 hold the lane's dims of two
      // tokens; element e of both goes into one packed pair (a byte
      // permute), and one packed dot with the two tokens' probabilities
      // adds both products (exact in float32) to acc[h][e]: half the
      // instructions of widening each value and multiplying it per head.
#pragma unroll
      for (int i = 0; i < NI; i += 2) {
        uint32_t pp[G];
#pragma unroll
        for (int h = 0; h < G; ++h)
          pp[h] = pack2<DT>(sc[(i * RPI + rsub) * G + h], sc[((i + 1) * RPI + rsub) * G + h]);
        const uint32_t va[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
        const uint32_t vb[4] = {vr[i + 1].x, vr[i + 1].y, vr[i + 1].z, vr[i + 1].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          // (token i, token i + 1) of elements 2k and 2k + 1
          const uint32_t lo = __builtin_amdgcn_perm(vb[k], va[k], 0x05040100u);
          const uint32_t hi = __builtin_amdgcn_perm(vb[k], va[k], 0x07060302u);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            acc[h][2 * k] = dot2<DT>(lo, pp[h], acc[h][2 * k]);
            acc[h][2 * k + 1] = dot2<DT>(hi, pp[h], acc[h][2 * k + 1]);
          }
        }
      }
    }
    // the next chunk's V goes in flight
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NI; ++i) vr[i] = vload(ad, i);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  }

  // the new row's slice of this head, to its slot (no other unit reads it)
  if (TAIL && tail_store && w == 0 && rsub == 0) {
    const size_t dst = (size_t)slot * row_bytes + lane_bytes;
    *reinterpret_cast<uint4*>(const_cast<char*>(kbase) + dst) = k_tail;
    *reinterpret_cast<uint4*>(const_cast<char*>(vbase) + dst) = v_tail;
  }

  // ---- epilogue: finish this wavefront's sums, merge wavefronts in LDS ----
#pragma unroll
  for (int m = G; m < 64; m <<= 1) l_run += shfl_xor_f(l_run, m);
#pragma unroll
  for (int m = LPR; m < 64; m <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] += shfl_xor_f(acc[h][e], m);
  if (lane < G) {
    s_ml[lane] = m_run;
    s_ml[G + lane] = l_run;
  }
  if (lane < LPR) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[h * D + e0 + e] = acc[h][e];
  }
  __syncthreads();

  merge_store<DT, D, G>(p, u, smem, S::LDS_FLOATS, SLOTS + G + 64, SLOTS + G + 64 + 2 * G, nw);
  });
}

// One workgroup of four wavefronts per (sequence, query head): merge the
// partials of sequences that span more than one non-empty partition, in one
// pass over them.  A partial row (D floats) is read as float4 by D/4 lanes,
// so a wavefront takes 64/(D/4) partitions per step and the four wavefronts
// interleave.  Each lane keeps a running maximum M, weight sum and weighted
// row, rescaled by 2^(M_old - M_new) when a partition raises M (the online
// softmax again, over partitions), so the loads of a partition's maximum,
// sum and row are issued together; lanes then combine through xor shuffles
// and LDS with one more rescale.
template <int DT, int D>
__global__ __launch_bounds__(256) void reduce_kernel(ReduceParams p) {
  constexpr int LPP = D / 4;     // lanes per partition row
  constexpr int PPW = 64 / LPP;  // partition rows per wavefront step
  constexpr int NWV = 4;
  typedef const __attribute__((address_space(4))) float cfloat;
  __shared__ float s_m[NWV];
  __shared__ float s_o[NWV][D];
  __shared__ float s_den[NWV];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int b = blockIdx.x / p.num_heads;
  const int hq = blockIdx.x % p.num_heads;
  const int L = min(p.context_lens[b], p.max_context_len);
  if (L <= 0) return;
  const int P = p.part;
  const int start = p.window > 0 ? max(0, L - p.window) : 0;
  const int p0 = start / P;
  const int p1 = (L - 1) / P;
  if (p0 == p1) return;
  const size_t base = ((size_t)b * p.num_heads + hq) * p.num_parts;
  cfloat* ml = (cfloat*)(p.max_logits + base);
  cfloat* es = (cfloat*)(p.exp_sums + base);

  const int sub = lane / LPP;  // which of the step's partitions
  const int dl = lane % LPP;   // float4 of the row
  float M = kNegInf, den = 0.0f;
  f32x4_t o = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const float* src = p.tmp_out + base * D + 4 * dl;
#pragma unroll 4
  for (int q = p0 + w * PPW + sub; q <= p1; q += NWV * PPW) {
    const float mq = ml[q];
    const float lq = es[q];
    const f32x4_t row = *reinterpret_cast<const f32x4_t*>(src + (size_t)q * D);
    const float Mn = fmaxf(M, mq);
    const float a = fast_exp2(M - Mn);   // 0 while M is still -inf
    const float wq = lq * fast_exp2(mq - Mn);
    den = den * a + wq;
    o = o * a + wq * row;
    M = Mn;
  }
  // lanes of one float4 column across the step's partitions, then waves
#pragma unroll
  for (int m = LPP; m < 64; m <<= 1) {
    const float Mo = shfl_xor_f(M, m);
    const float Mn = fmaxf(M, Mo);
    // a lane that saw no partition keeps M = -inf and zero sums
    const float a = Mn == kNegInf ? 0.0f : fast_exp2(M - Mn);
    const float ao = Mn == kNegInf ? 0.0f : fast_exp2(Mo - Mn);
    den = den * a + shfl_xor_f(den, m) * ao;
    f32x4_t oo;
    oo[0] = shfl_xor_f(o[0], m);
    oo[1] = shfl_xor_f(o[1], m);
    oo[2] = shfl_xor_f(o[2], m);
    oo[3] = shfl_xor_f(o[3], m);
    o = o * a + oo * ao;
    M = Mn;
  }
  if (sub == 0) {
    *reinterpret_cast<f32x4_t*>(&s_o[w][4 * dl]) = o;
    if (dl == 0) {
      s_m[w] = M;
      s_den[w] = den;
    }
  }
  __syncthreads();
  const float Mg = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
  float f[NWV];
  float tot = 0.0f;
#pragma unroll
  for (int v = 0; v < NWV; ++v) {
    f[v] = s_m[v] == kNegInf ? 0.0f : fast_exp2(s_m[v] - Mg);
    tot += s_den[v] * f[v];
  }
  const float inv = 1.0f / tot;
  for (int d = t; d < D; d += 256) {
    float v = 0.0f;
#pragma unroll
    for (int k = 0; k < NWV; ++k) v += s_o[k][d] * f[k];
    store_elem<DT>(p.out, ((size_t)b * p.num_heads + hq) * D + d, v * inv);
  }
}

}  // namespace pa
