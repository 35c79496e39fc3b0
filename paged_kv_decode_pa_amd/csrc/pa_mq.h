// Multi-query paged attention: a sequence brings n >= 1 new tokens (a prompt
// chunk, or a draft to verify), the last n of its L positions, and each new
// token attends causally to the keys up to its own position.
//
// Two paths share one plan kernel:
//   * per token: every query token runs as its own decode sequence (context
//     pos + 1, its sequence's block table) through the decode kernels; any
//     dtype and shape the decode path takes;
//   * tiled (16-bit KV, pages of 16+ tokens): the rows of a (sequence, KV
//     head) are the pairs (new token i, query head h of the group), numbered
//     f = i * G + h, and a wavefront takes R = 16 * NR consecutive rows as
//     the N side of the matrix-core tiles.  Each K/V chunk is then read once
//     for R rows instead of once per token, and every row masks the keys
//     past its own position.
//
// Tiled wavefront, per chunk of NT = 16 * TILES tokens inside one page:
//   q.k   S^T[t][r] = K[t][:] . Q[r][:] for each 16-row block (NR of them),
//         K fragments (A) loaded once for all blocks;
//   mask  row r keeps keys in [its window start, its position];
//   softmax per row, lanes c16 of a block own row c16 (4 lanes share it);
//   P.V   O^T[d][r] += V^T[d][t] . P^T[t][r], V^T gathered from the chunk in
//         LDS once per 16 dims for all row blocks.
// Workgroups hold 1..8 wavefronts that take a partition's chunks
// round-robin and merge in LDS; split-K partials use the decode layout, so
// the decode reduce merges them (each token's context is pos + 1).
#pragma once

#include <type_traits>

#include "pa_mfma.h"

namespace pa {

struct MQParams {
  void* out;                  // [T, Hq, D]
  float* tmp_out;             // [T, Hq, NP, D]
  float* max_logits;          // [T, Hq, NP], base-2 logits
  float* exp_sums;            // [T, Hq, NP]
  const int2* tiles;          // (sequence, first row) of each tile
  const int32_t* num_tiles;   // [2]: tiles, units
  const int2* units;          // (tile, partition) per grid unit, or null
  const void* q;              // [T, Hq, D]
  const void* k_cache;        // [NB, bs, Hkv, D]
  const void* v_cache;
  const int32_t* block_tables;  // [B, max_blocks_per_seq]
  const int32_t* context_lens;  // [B], counting every new token
  const int32_t* query_start;   // [B + 1]
  int max_blocks_per_seq;
  int max_context_len;
  int num_heads;
  int num_kv_heads;
  int group;                  // G = Hq / Hkv
  int num_blocks;
  int log2_bs;
  int window;
  int part;                   // partition size in tokens (> 0)
  int num_parts;
  int max_tiles;              // grid tiles per (KV head, partition)
  int num_tokens;             // T
  int resident_period;        // tiles per round of one workgroup per CU (0: plan order)
  int resident_span;          // tiles the chip holds at once
  int prio;                   // chunks per wave-priority step (0: none)
  float qk_mul;
  float cap_mul;
};

// Position -> plan tile when the whole grid is resident from the start.
// Workgroups i and i + period then share a CU for the whole launch (the
// dispatcher fills every CU once per round, in the same CU order each
// round), so plain longest-first order would put the longest tiles of every
// round on the same CUs.  Odd rounds take their tiles in reverse (a partial
// last round reverses what it has), so each CU pairs a long tile with a
// short one.  A grid larger than the chip keeps the plan order: its later
// workgroups go wherever a slot frees, longest first.
__device__ __forceinline__ int resident_tile(int i, int n, int period, int span) {
  if (period <= 0 || n > span) return i;
  const int r = i / period;
  if ((r & 1) == 0) return i;
  const int base = r * period;
  const int m = min(period, n - base);
  return base + (m - 1) - (i - base);
}

template <int DT, int D, int NR, int TILES, bool HEADS = false>
struct MQShape {
  static constexpr int R = 16 * NR;             // rows per wavefront
  static constexpr int NT = 16 * TILES;         // tokens per chunk
  static constexpr int KS = D / 32;             // q.k k-steps
  static constexpr int MT = D / 16;             // P.V tiles over head_dim
  static constexpr int VBYTES = NT * D * 2;     // V chunk in LDS
  static constexpr int VLOADS = VBYTES / 1024;  // 1 KB direct-to-LDS loads
  // LDS floats per wavefront: the two V chunks (after the loop, unless
  // HEADS: the [R][D] accumulators, rows padded to D + 4), the block-table
  // window, max and sum per row
  static constexpr int BUF = (HEADS || 2 * VBYTES / 4 > R * (D + 4)) ? 2 * VBYTES / 4 : R * (D + 4);
  static constexpr int TBL = BUF;
  static constexpr int ML = TBL + 64;
  static constexpr int LDS_FLOATS = ML + 2 * R;
  static_assert(VBYTES % 1024 == 0, "chunk must fill whole 1 KB LDS loads");
};

// HEADS: one wavefront per KV head, the workgroup holding one (tile,
// partition) unit for every head (a token's rows of all heads are adjacent in
// memory and get fetched together); each wavefront walks all chunks of its
// head and writes its rows from registers.  Otherwise the wavefronts split
// one head's chunks and merge in LDS.
template <int DT, int D, int NR, int TILES, bool HEADS = false>
__global__ __launch_bounds__(64 * kMaxWaves) void mq_mfma_kernel(MQParams p) {
  using S = MQShape<DT, D, NR, TILES, HEADS>;
  constexpr int R = S::R, NT = S::NT, KS = S::KS, MT = S::MT, VLOADS = S::VLOADS;
  constexpr int EB = 2;
  typedef const __attribute__((address_space(4))) int32_t cint32;
  typedef const __attribute__((address_space(4))) uint64_t cu64;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int c16 = lane & 15;
  const int j = lane >> 4;

  extern __shared__ __align__(16) float smem[];
  float* s_wave = smem + w * S::LDS_FLOATS;
  char* vbuf = reinterpret_cast<char*>(s_wave);
  int32_t* tbl = reinterpret_cast<int32_t*>(s_wave + S::TBL);

  // unit: KV head fastest (or the wavefront's head), then tiles (a
  // sequence's tiles side by side, so they share its pages in L2), then
  // partitions
  // kernel arguments along the unit's lookup chain (tile, sequence start
  // and length), read in one round, the loads of each link issued together
  asm volatile("" ::"s"(p.num_kv_heads), "s"(p.num_tiles), "s"(p.tiles), "s"(p.max_tiles),
               "s"(p.resident_period), "s"(p.resident_span), "s"(p.query_start),
               "s"(p.context_lens), "s"(p.num_tokens), "s"(p.max_context_len), "s"(p.group),
               "s"(p.window), "s"(p.part), "s"(p.q), "s"(p.num_heads), "s"(p.block_tables),
               "s"(p.max_blocks_per_seq), "s"(p.log2_bs), "s"(p.k_cache), "s"(p.v_cache),
               "s"(p.num_blocks), "s"(nw));
  const int Hq = p.num_heads;
  const int G = p.group;
  const int g = HEADS ? w : (int)(blockIdx.x % p.num_kv_heads);
  const int rest = HEADS ? (int)blockIdx.x : (int)(blockIdx.x / p.num_kv_heads);
  const int cw = HEADS ? 0 : w;       // first chunk of this wavefront
  const int cstride = HEADS ? 1 : nw;  // its chunk stride
  const int part = rest / p.max_tiles;
  const int n_tiles = *(cint32*)p.num_tiles;
  if (rest % p.max_tiles >= n_tiles) return;
  const int tile = resident_tile(rest % p.max_tiles, n_tiles, p.resident_period, p.resident_span);
  const uint64_t tl = ((cu64*)p.tiles)[tile];
  const int b = (int)(uint32_t)tl;
  const int f0 = (int)(uint32_t)(tl >> 32);
  // the sequence's rows, clamped to [0, T) whatever query_start holds
  const int qs_b = ((cint32*)p.query_start)[b];
  const int qs_b1 = ((cint32*)p.query_start)[b + 1];
  const int L_raw = ((cint32*)p.context_lens)[b];
  asm volatile("" ::"s"(qs_b), "s"(qs_b1), "s"(L_raw));  // one round for the three
  const int q0 = min(max(qs_b, 0), p.num_tokens);
  const int n = min(max(qs_b1 - q0, 0), p.num_tokens - q0);
  const int f_end = min(f0 + R, n * G);
  const int L = min(L_raw, p.max_context_len);
  const int W = p.window;
  const int P = p.part;
  auto key_lo = [&](int pos) { return W > 0 ? max(0, pos + 1 - W) : 0; };
  const int i_first = f0 / G;
  const int i_last = (f_end - 1) / G;
  const int lo = max(key_lo(L - n + i_first), part * P);
  const int hi = min(L - n + i_last + 1, part * P + P);
  if (f0 >= f_end || lo >= hi) return;

  // this lane's rows (one per 16-row block): keys it attends to within the
  // unit, and its query fragments (B operand of q.k; zero for rows past the
  // sequence's last)
  int a_lo[NR], a_hi[NR];
  uint4 qf[NR][KS];
#pragma unroll
  for (int nb = 0; nb < NR; ++nb) {
    const int f = f0 + 16 * nb + c16;
    const bool act = f < f_end;
    const int i = act ? f / G : i_first;
    const int h = act ? f - i * G : 0;
    const int pos = L - n + i;
    a_lo[nb] = act ? max(lo, key_lo(pos)) : 0;
    a_hi[nb] = act ? min(hi, pos + 1) : 0;
    const char* qb = static_cast<const char*>(p.q) +
                     (((size_t)(q0 + i) * Hq + (size_t)g * G + h) * D + 8 * j) * EB;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[nb][s] = act ? ld16(qb + (size_t)s * 32 * EB) : make_uint4(0, 0, 0, 0);
  }

  // keys every active row attends to: chunks inside need no mask (rows past
  // the sequence's end are never written, whatever they accumulate)
  const int full_lo = max(lo, key_lo(L - n + (min(f0 + R, f_end) - 1) / G));
  const int full_hi = min(hi, L - n + f0 / G + 1);

  const int32_t* bt = p.block_tables + (size_t)b * p.max_blocks_per_seq;
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

  const uint32_t row_bytes = (uint32_t)(p.num_kv_heads * D * EB);
  const uint32_t page_bytes = row_bytes << log2_bs;
  const uint32_t head_bytes = (uint32_t)(g * D * EB);
  const char* kbase = static_cast<const char*>(p.k_cache);
  const char* vbase = static_cast<const char*>(p.v_cache);
  // prefetch target past the last chunk: the tile's first query row (the
  // descriptor's bounds turn anything beyond it into zeros)
  const char* dummy = static_cast<const char*>(p.q) +
                      ((size_t)(q0 + i_first) * Hq + (size_t)g * G) * D * EB;

  // V copy: instruction i moves LDS bytes [1024 i, 1024 i + 1024); lane l's
  // 16 bytes hold row r, stored segment sg ^ f(r) of global segment sg
  int v_row[VLOADS];
  uint32_t v_seg_bytes[VLOADS];
#pragma unroll
  for (int i = 0; i < VLOADS; ++i) {
    const int o = i * 1024 + lane * 16;
    const int r = o / (2 * D);
    const int sg = ((o % (2 * D)) >> 4) ^ v_swz<D>(r);
    v_row[i] = r;
    v_seg_bytes[i] = head_bytes + (uint32_t)(sg * 16);
  }

  struct Addr {
    rsrc_t kr, vr;
    uint32_t soff;
    int rlo, rhi;
  };
  auto chunk_addr = [&](int c, Addr& a) {
    const int cs = c * NT;
    const int cpg = max(cs, lo) >> log2_bs;
    if (cpg < pg0 || cpg - pg0 >= 64) refill(cpg);
    int phys = __builtin_amdgcn_readfirstlane(tbl[cpg - pg0]);
    phys = ((unsigned)phys < (unsigned)p.num_blocks) ? phys : 0;
    const uint64_t base = (uint64_t)phys * page_bytes;
    a.kr = make_rsrc(kbase + base, page_bytes);
    a.vr = make_rsrc(vbase + base, page_bytes);
    a.soff = (uint32_t)(cs & ((1 << log2_bs) - 1)) * row_bytes;
    a.rlo = lo - cs;
    a.rhi = hi - 1 - cs;
  };
  auto dummy_addr = [&](Addr& a) {
    a.kr = make_rsrc(dummy, (uint32_t)(G * D * EB));
    a.vr = a.kr;
    a.soff = 0;
    a.rlo = 0;
    a.rhi = 0;
  };
  // K loads of tile t, k-step s, whole lines (kline_rowseg)
  auto kload = [&](const Addr& a, int t, int s) -> uint4 {
    int row, seg;
    kline_rowseg(c16, j, t, s, row, seg);
    const int r = min(max(row, a.rlo), a.rhi);
    return ld16_buf(a.kr, (uint32_t)r * row_bytes + head_bytes + (uint32_t)(seg * 16), a.soff);
  };
  auto vcopy = [&](const Addr& a, char* vb) {
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int r = min(max(v_row[i], a.rlo), a.rhi);
      ld16_buf_to_lds(a.vr, vb + i * 1024, (uint32_t)r * row_bytes + v_seg_bytes[i], a.soff);
    }
  };

  float m_run[NR], l_run[NR];
  f32x4_t acc[NR][MT];
#pragma unroll
  for (int nb = 0; nb < NR; ++nb) {
    m_run[nb] = kNegInf;
    l_run[nb] = 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nb][mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  const int c0 = lo / NT;
  const int c1 = (hi - 1) / NT;
  constexpr int NK = TILES * KS;
  constexpr int NV = VLOADS;
  auto addr_of = [&](int cc, Addr& a) {
    if (cc <= c1) chunk_addr(cc, a);
    else dummy_addr(a);
  };
  auto issue_k = [&](const Addr& a, uint4 (&k)[TILES][KS]) {
#pragma unroll
    for (int t = 0; t < TILES; ++t)
#pragma unroll
      for (int s = 0; s < KS; ++s) k[t][s] = kload(a, t, s);
  };

  // One chunk cc, then its K slot and V buffer are refilled with chunk cn.
  auto step = [&](int cc, int cn, uint4 (&k)[TILES][KS], char* vb) __attribute__((always_inline)) {
    f32x4_t sc[NR][TILES];
#pragma unroll
    for (int nb = 0; nb < NR; ++nb)
#pragma unroll
      for (int t = 0; t < TILES; ++t) sc[nb][t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < TILES; ++t)
#pragma unroll
      for (int s = 0; s < KS; s += 2) {
        uint4 a0, a1;
        kline_operands(c16, k[t][s], k[t][s + 1], a0, a1);
#pragma unroll
        for (int nb = 0; nb < NR; ++nb) {
          sc[nb][t] = mfma_k32<DT>(a0, qf[nb][s], sc[nb][t]);
          sc[nb][t] = mfma_k32<DT>(a1, qf[nb][s + 1], sc[nb][t]);
        }
      }
    __builtin_amdgcn_sched_barrier(0);
    Addr an;
    addr_of(cn, an);
    issue_k(an, k);
    __builtin_amdgcn_sched_barrier(0);

    const int cs = cc * NT;
    uint32_t pk[NR][2 * TILES];
#pragma unroll
    for (int nb = 0; nb < NR; ++nb) {
      float pr[TILES][4];
      if (p.cap_mul > 0.0f) {
#pragma unroll
        for (int t = 0; t < TILES; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) pr[t][i] = p.cap_mul * tanh_def(sc[nb][t][i] * p.qk_mul);
      } else {
#pragma unroll
        for (int t = 0; t < TILES; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) pr[t][i] = sc[nb][t][i] * p.qk_mul;
      }
      float cmax = kNegInf;
      if (cs < full_lo || cs + NT > full_hi) {  // keys some row of the wavefront must not see
#pragma unroll
        for (int t = 0; t < TILES; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int pos = cs + 16 * t + 4 * j + i;
            pr[t][i] = (pos >= a_lo[nb] && pos < a_hi[nb]) ? pr[t][i] : kNegInf;
          }
      }
#pragma unroll
      for (int t = 0; t < TILES; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) cmax = fmaxf(cmax, pr[t][i]);
      cmax = fmaxf(cmax, shfl_xor_f(cmax, 16));
      cmax = fmaxf(cmax, shfl_xor_f(cmax, 32));
      const float m_new = fmaxf(m_run[nb], cmax);
      // a row with no key yet keeps (-inf, 0, 0): exponents against 0
      const float m_use = m_new == kNegInf ? 0.0f : m_new;
      const float alpha = fast_exp2(m_run[nb] - m_use);
      float psum = 0.0f;
#pragma unroll
      for (int t = 0; t < TILES; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr[t][i] = fast_exp2(pr[t][i] - m_use);
          psum += pr[t][i];
        }
      l_run[nb] = l_run[nb] * alpha + psum;
      m_run[nb] = m_new;
      if (any_rescale(alpha)) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[nb][mt] *= alpha;
      }
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        pk[nb][2 * t] = pack2<DT>(pr[t][0], pr[t][1]);
        pk[nb][2 * t + 1] = pack2<DT>(pr[t][2], pr[t][3]);
      }
    }

    __builtin_amdgcn_s_waitcnt(vmcnt_only(2 * NK + NV));
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      uint32_t vv[2 * TILES];
      vt_frag<D, TILES>(vb, mt, c16, j, vv);
#pragma unroll
      for (int nb = 0; nb < NR; ++nb) {
        if constexpr (TILES == 2)
          acc[nb][mt] = mfma_k32<DT>(make_uint4(vv[0], vv[1], vv[2], vv[3]),
                                     make_uint4(pk[nb][0], pk[nb][1], pk[nb][2], pk[nb][3]),
                                     acc[nb][mt]);
        else
          acc[nb][mt] = mfma_k16<DT>(make_uint2(vv[0], vv[1]), make_uint2(pk[nb][0], pk[nb][1]),
                                     acc[nb][mt]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    __builtin_amdgcn_sched_barrier(0);
    vcopy(an, vb);
    __builtin_amdgcn_sched_barrier(0);
  };

  uint4 kf0[TILES][KS], kf1[TILES][KS];
  char* vb0 = vbuf;
  char* vb1 = vbuf + S::VBYTES;
  int c = c0 + cw;
  if (c <= c1) {
    Addr a;
    addr_of(c, a);
    issue_k(a, kf0);
    __builtin_amdgcn_sched_barrier(0);
    vcopy(a, vb0);
    __builtin_amdgcn_sched_barrier(0);
    addr_of(c + cstride, a);
    issue_k(a, kf1);
    __builtin_amdgcn_sched_barrier(0);
    vcopy(a, vb1);
    __builtin_amdgcn_sched_barrier(0);
    // the two V buffers as restrict pointers: the compiler's own wait before
    // one buffer's LDS reads then leaves the other buffer's copy in flight
    // (the explicit wait in step covers what the reads need)
    auto two = [&](char* __restrict__ b0, char* __restrict__ b1) __attribute__((always_inline)) {
      step(c, c + 2 * cstride, kf0, b0);
      step(c + cstride, c + 3 * cstride, kf1, b1);
    };
#pragma clang loop unroll(disable)
    for (; c <= c1; c += 2 * cstride) {
      // issue priority from the chunks this wavefront has left, in steps of
      // p.prio chunks: the wavefronts sharing a SIMD are otherwise served
      // oldest first, so a CU's older workgroup would finish long before
      // the younger one, which then runs alone
      if (p.prio) {
        const int rem = (c1 - c) / cstride;
        if (rem >= 4 * p.prio) __builtin_amdgcn_s_setprio(3);
        else if (rem >= 2 * p.prio) __builtin_amdgcn_s_setprio(2);
        else if (rem >= p.prio) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
      }
      two(vb0, vb1);
    }
  }
  // drain the trailing loads (the V buffers are reused below)
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  if constexpr (HEADS) {
    // the wavefront holds its head's whole unit: write its rows directly
#pragma unroll
    for (int nb = 0; nb < NR; ++nb) {
      float l = l_run[nb];
      l += shfl_xor_f(l, 16);
      l += shfl_xor_f(l, 32);
      const int f = f0 + 16 * nb + c16;
      if (f >= f_end || l == 0.0f) continue;  // past the end, or no key here
      const float inv = 1.0f / l;
      const int i = f / G;
      const int h = f - i * G;
      const int pos = L - n + i;
      const size_t row = (size_t)(q0 + i) * Hq + (size_t)g * G + h;
      if (key_lo(pos) / P == pos / P) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const size_t e = row * D + 16 * mt + 4 * j;
          const uint2 v = make_uint2(pack2<DT>(acc[nb][mt][0] * inv, acc[nb][mt][1] * inv),
                                     pack2<DT>(acc[nb][mt][2] * inv, acc[nb][mt][3] * inv));
          *reinterpret_cast<uint2*>(static_cast<char*>(p.out) + e * EB) = v;
        }
      } else {
        const size_t pi = row * p.num_parts + part;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          *reinterpret_cast<f32x4_t*>(p.tmp_out + pi * D + 16 * mt + 4 * j) = acc[nb][mt] * inv;
        if (j == 0) {
          p.max_logits[pi] = m_run[nb];
          p.exp_sums[pi] = l;
        }
      }
    }
    return;
  }

  // ---- epilogue: per-row sums over the four lanes, staged in LDS ----
  float* s_acc = s_wave;
  float* s_ml = s_wave + S::ML;
#pragma unroll
  for (int nb = 0; nb < NR; ++nb) {
    float l = l_run[nb];
    l += shfl_xor_f(l, 16);
    l += shfl_xor_f(l, 32);
    const int r = 16 * nb + c16;
    if (j == 0) {
      s_ml[r] = m_run[nb];
      s_ml[R + r] = l;
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      *reinterpret_cast<f32x4_t*>(s_acc + r * acc_stride<D>() + 16 * mt + 4 * j) = acc[nb][mt];
  }
  __syncthreads();

  // merge the wavefronts and write each row: the output when the row's keys
  // all lie in this partition, else its split-K partial
  for (int e = threadIdx.x; e < R * D; e += blockDim.x) {
    const int r = e / D;
    const int d = e % D;
    const int f = f0 + r;
    if (f >= f_end) break;  // rows are in order: the rest are past the end
    float M = kNegInf;
    for (int v = 0; v < nw; ++v) M = fmaxf(M, smem[v * S::LDS_FLOATS + S::ML + r]);
    if (M == kNegInf) continue;  // no key of this row in the partition
    float den = 0.0f, num = 0.0f;
    for (int v = 0; v < nw; ++v) {
      const float* lv = smem + v * S::LDS_FLOATS;
      const float fct = fast_exp2(lv[S::ML + r] - M);
      den += fct * lv[S::ML + R + r];
      num += fct * lv[r * acc_stride<D>() + d];
    }
    const int i = f / G;
    const int h = f - i * G;
    const int pos = L - n + i;
    const size_t row = (size_t)(q0 + i) * Hq + (size_t)g * G + h;
    if (key_lo(pos) / P == pos / P) {
      store_elem<DT>(p.out, row * D + d, num / den);
    } else {
      const size_t pi = row * p.num_parts + part;
      p.tmp_out[pi * D + d] = num / den;
      if (d == 0) {
        p.max_logits[pi] = M;
        p.exp_sums[pi] = den;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Workgroup-shared variant for many rows per (sequence, KV head): prompt
// chunks and whole-prompt prefill.  Four wavefronts own consecutive 16 * NR
// row blocks of one R = 64 * NR row tile and walk the same keys in lockstep:
// each K and V chunk is copied HBM -> LDS once (the four wavefronts issue a
// quarter of the direct-to-LDS loads each) and read by all of them, so the
// pages are fetched once per R rows.  NBUF chunk buffers keep NBUF - 1
// chunks in flight; one workgroup barrier per chunk publishes the next one.
//   q.k  A = K fragments from LDS (16-byte reads; K rows stored with their
//        16-byte segments XOR-swizzled so 16 rows hit distinct banks);
//   P.V  A = V^T gathered from LDS as in the per-wavefront kernel.
// A wavefront skips the arithmetic of chunks none of its rows attends to
// (the causal upper triangle), but still loads and syncs.
template <int DT, int D, int NR, int TILES, int NBUF_ = 3>
struct MQWGShape {
  static constexpr int NW = 4;                  // wavefronts per workgroup
  static constexpr int RW = 16 * NR;            // rows per wavefront
  static constexpr int R = NW * RW;             // rows per workgroup
  static constexpr int NT = 16 * TILES;         // tokens per chunk
  static constexpr int KS = D / 32;
  static constexpr int MT = D / 16;
  static constexpr int CBYTES = NT * D * 2;     // one K or V chunk
  static constexpr int LOADS = CBYTES / 1024;   // 1 KB loads per K or V chunk
  static constexpr int LPW = 2 * LOADS / NW;    // K + V loads per wavefront per chunk
  static constexpr int NBUF = NBUF_;              // chunk buffers (NBUF - 1 in flight)
  static_assert(CBYTES % 1024 == 0 && (2 * LOADS) % NW == 0, "chunk shape");
};

// How far (base-2 logit units) a row's logits may pass its reference
// maximum before the shared kernel moves it and rescales the accumulators.
// The reference is exact for the result (sum, accumulators and a partial's
// max all use it); only the probabilities grow, below 2^kMaxSlack, which the
// 16-bit P operand and fp32 sums hold without loss of relative precision.
// Most chunks then skip the rescale.
constexpr float kMaxSlack = 8.0f;
constexpr float kSlackPow = 256.0f;  // 2^kMaxSlack

// f(integral_constant<K>), f(integral_constant<K + 1>), ... up to N - 1
template <int K, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (K < N) {
    f(std::integral_constant<int, K>{});
    static_for<K + 1, N>(f);
  }
}

// K rows in LDS: 16-byte segment s of row r is stored at s ^ k_swz(r)
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  return D >= 128 ? (r & 15) : ((r >> 1) & 7);
}

// Workgroups per CU the shapes the library picks (a wavefront's rows x
// dims at most 128, or head_dim 256 with one row block) are compiled for:
// as many as their LDS allows, at most 4 (registers 128 per lane then).
template <int D, int NR, int TILES, int NBUF>
constexpr int mq_wg_min_blocks() {
  constexpr int by_lds = 160 * 1024 / (NBUF * 2 * 16 * TILES * D * 2);
  return (NR * D <= 128 || (D == 256 && NR == 1)) ? (by_lds < 4 ? by_lds : 4) : 1;
}

template <int DT, int D, int NR, int TILES, int NBUF_>
__global__ __launch_bounds__(256, (mq_wg_min_blocks<D, NR, TILES, NBUF_>())) void mq_wg_kernel(
    MQParams p) {
  using S = MQWGShape<DT, D, NR, TILES, NBUF_>;
  constexpr int NW = S::NW, RW = S::RW, R = S::R, NT = S::NT, KS = S::KS, MT = S::MT;
  constexpr int CBYTES = S::CBYTES, LOADS = S::LOADS, LPW = S::LPW, NBUF = S::NBUF;
  constexpr int EB = 2;
  typedef const __attribute__((address_space(4))) int32_t cint32;
  typedef const __attribute__((address_space(4))) uint64_t cu64;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15;
  const int j = lane >> 4;
  // The chunk buffers, each its own LDS object.  Up to head_dim 128 the
  // chunk loop is unrolled over them: every LDS address is then a lane
  // offset plus a constant, and the compiler's wait before a read of one
  // buffer counts only the copies into that one.  At head_dim 256 the lane
  // offsets of 24 fragments would stay live in registers, so the loop takes
  // one chunk a step, the buffers slices of one array picked at run time
  // (the restrict pointers of each step then keep the compiler's waits to
  // the copies into the buffer read).
  constexpr bool kUnroll = D <= 128;
  constexpr int kOwn = kUnroll ? 2 * CBYTES : 16;
  __shared__ __align__(16) char lds_b0[kUnroll ? 2 * CBYTES : NBUF * 2 * CBYTES];
  __shared__ __align__(16) char lds_b1[kOwn];
  __shared__ __align__(16) char lds_b2[kOwn];
  __shared__ __align__(16) char lds_b3[NBUF == 4 ? kOwn : 16];
  static_assert(NBUF == 3 || NBUF == 4, "three or four chunk buffers");
  auto buf = [&](auto kc) __attribute__((always_inline)) -> char* {
    constexpr int k = decltype(kc)::value % NBUF;
    if constexpr (!kUnroll) return lds_b0 + k * 2 * CBYTES;
    else if constexpr (k == 0) return lds_b0;
    else if constexpr (k == 1) return lds_b1;
    else if constexpr (k == 2) return lds_b2;
    else return lds_b3;
  };

  const int Hq = p.num_heads;
  const int G = p.group;
  // unit: KV head fastest, then the plan's (tile, partition) list, or
  // without one tiles in plan order with partitions slowest
  // The unit's lookups form a chain (list entry, tile, sequence start and
  // length); the kernel arguments along it are read in one round here, and
  // the loads of each link are issued together.  Left to the compiler, the
  // arguments came in rounds of their own between the links.
  asm volatile("" ::"s"(p.num_kv_heads), "s"(p.units), "s"(p.num_tiles), "s"(p.tiles),
               "s"(p.max_tiles), "s"(p.query_start), "s"(p.context_lens), "s"(p.num_tokens),
               "s"(p.max_context_len), "s"(p.group), "s"(p.window), "s"(p.part), "s"(p.q),
               "s"(p.num_heads), "s"(p.block_tables), "s"(p.max_blocks_per_seq),
               "s"(p.log2_bs), "s"(p.k_cache), "s"(p.v_cache), "s"(p.num_blocks));
  const int g = blockIdx.x % p.num_kv_heads;
  const int rest = blockIdx.x / p.num_kv_heads;
  int tile, part;
  const int n_tiles = *(cint32*)p.num_tiles;
  if (p.units != nullptr) {
    // the entry is read with the list's length: the list has room for an
    // entry at every position of the grid, written or not
    const int n_units = ((cint32*)p.num_tiles)[1];
    const uint64_t u = ((cu64*)p.units)[rest];
    asm volatile("" ::"s"(n_units), "s"(u), "s"(n_tiles));  // one round for the three
    if (rest >= n_units) return;
    tile = (int)(uint32_t)u;
    part = (int)(uint32_t)(u >> 32);
    if (tile >= n_tiles) return;
  } else {
    tile = rest % p.max_tiles;
    part = rest / p.max_tiles;
    if (tile >= n_tiles) return;
  }
  const uint64_t tl = ((cu64*)p.tiles)[tile];
  const int b = (int)(uint32_t)tl;
  const int f0 = (int)(uint32_t)(tl >> 32);
  const int qs_b = ((cint32*)p.query_start)[b];
  const int qs_b1 = ((cint32*)p.query_start)[b + 1];
  const int L_raw = ((cint32*)p.context_lens)[b];
  asm volatile("" ::"s"(qs_b), "s"(qs_b1), "s"(L_raw));  // one round for the three
  const int q0 = min(max(qs_b, 0), p.num_tokens);
  const int n = min(max(qs_b1 - q0, 0), p.num_tokens - q0);
  const int f_end = min(f0 + R, n * G);
  const int L = min(L_raw, p.max_context_len);
  const int W = p.window;
  const int P = p.part;
  auto key_lo = [&](int pos) { return W > 0 ? max(0, pos + 1 - W) : 0; };
  const int i_first = f0 / G;
  const int i_last = (f_end - 1) / G;
  const int lo = max(key_lo(L - n + i_first), part * P);
  const int hi = min(L - n + i_last + 1, part * P + P);
  if (f0 >= f_end || lo >= hi) return;  // uniform over the workgroup

  // this wavefront's rows: f0 + RW * w + 16 nb + c16
  const int fw0 = f0 + RW * w;
  // a row's keys [a_lo, a_hi), less the lane's key offset 4 j in a chunk
  int a_lo[NR], a_hi[NR];
  uint4 qf[NR][KS];
#pragma unroll
  for (int nb = 0; nb < NR; ++nb) {
    const int f = fw0 + 16 * nb + c16;
    const bool act = f < f_end;
    const int i = act ? f / G : i_first;
    const int h = act ? f - i * G : 0;
    const int pos = L - n + i;
    a_lo[nb] = (act ? max(lo, key_lo(pos)) : 0) - 4 * j;
    a_hi[nb] = (act ? min(hi, pos + 1) : 0) - 4 * j;
    const char* qb = static_cast<const char*>(p.q) +
                     (((size_t)(q0 + i) * Hq + (size_t)g * G + h) * D + 8 * j) * EB;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[nb][s] = act ? ld16(qb + (size_t)s * 32 * EB) : make_uint4(0, 0, 0, 0);
  }
  // keys this wavefront attends to at all (empty when it has no rows), and
  // keys all its rows attend to (chunks inside need no mask)
  int wlo = hi, whi = lo, full_lo = hi, full_hi = lo;
  if (fw0 < f_end) {
    const int fl = min(fw0 + RW, f_end) - 1;
    wlo = max(lo, key_lo(L - n + fw0 / G));
    whi = min(hi, L - n + fl / G + 1);
    full_lo = max(lo, key_lo(L - n + fl / G));
    full_hi = min(hi, L - n + fw0 / G + 1);
  }

  const int32_t* bt = p.block_tables + (size_t)b * p.max_blocks_per_seq;
  const int log2_bs = p.log2_bs;
  const int last_pg = (hi - 1) >> log2_bs;
  // 64 consecutive block-table entries, one per lane, read by lane index
  int pg0 = -(1 << 30);
  int tbl_v = 0;
  const uint32_t row_bytes = (uint32_t)(p.num_kv_heads * D * EB);
  const uint32_t page_bytes = row_bytes << log2_bs;
  const uint32_t head_bytes = (uint32_t)(g * D * EB);
  const char* kbase = static_cast<const char*>(p.k_cache);
  const char* vbase = static_cast<const char*>(p.v_cache);
  const char* dummy = static_cast<const char*>(p.q) +
                      ((size_t)(q0 + i_first) * Hq + (size_t)g * G) * D * EB;

  // this wavefront's share of a chunk's copies: loads q = LPW * w + k; the
  // first LOADS are K, the rest V.  Lane l's 16 bytes land at byte
  // 1024 (q % LOADS) + 16 l of the K or V chunk: row r, stored segment
  // sg, global segment sg ^ swizzle(r).
  // Four 16-token tiles a chunk (64 keys) span two 32-token pages: a
  // wavefront's LPW = LOADS / 2 loads then cover one 32-row half of K
  // (wavefronts 0, 1) or V (2, 3), addressed from that half's own page.
  constexpr bool kTwoPages = TILES == 4;
  static_assert(!kTwoPages || LPW * 2 == LOADS, "a wavefront's loads cover one half chunk");
  uint32_t ld_off[LPW];
#pragma unroll
  for (int k = 0; k < LPW; ++k) {
    const int q = LPW * w + k;
    const int o = (q % LOADS) * 1024 + lane * 16;
    const int r = o / (2 * D);
    const int sg = (o % (2 * D)) >> 4;
    const int r_src = kTwoPages ? r % (NT / 2) : r;  // row in the half's page
    ld_off[k] = (uint32_t)r_src * row_bytes + head_bytes +
                (uint32_t)((sg ^ (q < LOADS ? k_swz<D>(r) : v_swz<D>(r))) * 16);
  }
  // The copies of chunk c: the descriptors start at the chunk's first row
  // and end after its last key (hi - 1), so that rows past it (not yet
  // written, or another sequence's) read as zeros: their keys are masked
  // and their V rows then add nothing.  Rows before the first key (lo) are
  // earlier positions of the sequence, finite, and masked too.
  auto issue = [&](int c, char* kb) {
    if constexpr (kTwoPages) {
      // this wavefront's half: rows [cs, cs + NT / 2) of one page (the
      // launch takes four tiles a chunk only over 32-token pages); a half
      // with no key in [lo, hi) reads as zeros, as rows past hi do
      const int cs = c * NT + (w & 1) * (NT / 2);
      rsrc_t r = make_rsrc(dummy, 0u);
      if (cs < hi && cs + NT / 2 > lo) {
        const int cpg = cs >> log2_bs;
        if (cpg < pg0 || cpg - pg0 >= 64) {
          pg0 = cpg;
          const int pg = cpg + lane;
          tbl_v = pg <= last_pg ? bt[pg] : 0;
          __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
        }
        int phys = __builtin_amdgcn_readlane(tbl_v, cpg - pg0);
        phys = ((unsigned)phys < (unsigned)p.num_blocks) ? phys : 0;
        r = make_rsrc((w < 2 ? kbase : vbase) + (uint64_t)phys * page_bytes,
                      (uint32_t)min(hi - cs, NT / 2) * row_bytes);
      }
#pragma unroll
      for (int k = 0; k < LPW; ++k) {
        const int q = LPW * w + k;
        ld16_buf_to_lds(r, kb + (q < LOADS ? 0 : CBYTES) + (q % LOADS) * 1024, ld_off[k], 0);
      }
      return;
    }
    rsrc_t kr, vr;
    if (c * NT < hi) {
      const int cs = c * NT;
      const int cpg = max(cs, lo) >> log2_bs;
      if (cpg < pg0 || cpg - pg0 >= 64) {
        pg0 = cpg;
        const int pg = cpg + lane;
        tbl_v = pg <= last_pg ? bt[pg] : 0;
        // (every 64 pages) wait here: a load still pending where the paths
        // join would make the compiler wait for every copy in flight on
        // each chunk
        __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
      }
      int phys = __builtin_amdgcn_readlane(tbl_v, cpg - pg0);
      phys = ((unsigned)phys < (unsigned)p.num_blocks) ? phys : 0;
      const uint64_t base = (uint64_t)phys * page_bytes +
                            (uint32_t)(cs & ((1 << log2_bs) - 1)) * row_bytes;
      const uint32_t bytes = (uint32_t)min(hi - cs, NT) * row_bytes;
      kr = make_rsrc(kbase + base, bytes);
      vr = make_rsrc(vbase + base, bytes);
    } else {
      kr = make_rsrc(dummy, (uint32_t)(G * D * EB));
      vr = kr;
    }
#pragma unroll
    for (int k = 0; k < LPW; ++k) {
      const int q = LPW * w + k;
      const bool is_k = q < LOADS;
      ld16_buf_to_lds(is_k ? kr : vr, kb + (is_k ? 0 : CBYTES) + (q % LOADS) * 1024, ld_off[k], 0);
    }
  };

  float m_run[NR], l_run[NR], nm[NR];
  f32x4_t acc[NR][MT];
#pragma unroll
  for (int nb = 0; nb < NR; ++nb) {
    m_run[nb] = kNegInf;
    nm[nb] = 0.0f;
    l_run[nb] = 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nb][mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  const int c0 = lo / NT;
  const int c1 = (hi - 1) / NT;
  // the chunk holding the first key of this wavefront's last row: every
  // row's first keys lie at or before it (a row's first key does not
  // decrease with its position)
  const int c_ref = full_lo / NT;
  static_for<0, NBUF - 1>([&](auto kc) __attribute__((always_inline)) {
    issue(c0 + decltype(kc)::value, buf(kc));
  });
  // Chunk c from buffer kb; next (chunk c - 1's buffer) takes chunk
  // c + NBUF - 1.  This wavefront's copies of chunk c are done at the wait;
  // the barrier makes every wavefront's copies visible and puts every
  // wavefront past chunk c - 1.  That wait and barrier are all the ordering
  // the copies need: the barrier carries no release fence (which would wait
  // for every copy in flight), and kb and next are restrict, so the
  // compiler's own wait before the LDS reads does not cover the copy just
  // issued into the other buffer.
  auto chunk = [&](int c, const char* __restrict__ kb, char* __restrict__ next, auto capped_c)
                   __attribute__((always_inline)) {
    constexpr bool capped = decltype(capped_c)::value;
    __builtin_amdgcn_s_waitcnt(vmcnt_only((NBUF - 2) * LPW));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    issue(c + NBUF - 1, next);
    const char* vb = kb + CBYTES;
    const int cs = c * NT;
    if (wlo >= whi || cs + NT <= wlo || cs >= whi) return;  // no row of this wavefront looks here

    f32x4_t sc[NR][TILES];
#pragma unroll
    for (int nb = 0; nb < NR; ++nb)
#pragma unroll
      for (int t = 0; t < TILES; ++t) sc[nb][t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < TILES; ++t)
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int r = 16 * t + c16;
        const uint4 kf = *reinterpret_cast<const uint4*>(
            kb + r * 2 * D + (((4 * s + j) ^ k_swz<D>(r)) << 4));
#pragma unroll
        for (int nb = 0; nb < NR; ++nb) sc[nb][t] = mfma_k32<DT>(kf, qf[nb][s], sc[nb][t]);
      }

    uint32_t pk[NR][2 * TILES];
#pragma unroll
    for (int nb = 0; nb < NR; ++nb) {
      // logits in base-2 units are pr * smul: soft-capped ones come out of
      // the cap already scaled, plain ones keep the scale for the exponent's
      // fma below
      float pr[TILES][4];
      const float smul = capped ? 1.0f : p.qk_mul;
      if constexpr (capped) {
#pragma unroll
        for (int t = 0; t < TILES; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) pr[t][i] = p.cap_mul * tanh_def(sc[nb][t][i] * p.qk_mul);
      } else {
#pragma unroll
        for (int t = 0; t < TILES; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) pr[t][i] = sc[nb][t][i];
      }
      if (cs < full_lo || cs + NT > full_hi) {  // keys some row of the wavefront must not see
        // key 16 t + 4 j + i of the chunk, against the row's bounds less cs + 4 j
        const int klo = a_lo[nb] - cs;
        const int khi = a_hi[nb] - cs;
#pragma unroll
        for (int t = 0; t < TILES; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            pr[t][i] = (16 * t + i >= klo && 16 * t + i < khi) ? pr[t][i] : kNegInf;
      }
      // Probabilities against the row's reference maximum (exponent base
      // nm = -reference; 0 for a row with no key yet).  The reference moves
      // only when a logit passes it by more than kMaxSlack, so most chunks
      // keep these: the exact maximum is taken (max over the chunk, then
      // over the row's four lanes) only in the chunks that hold some row's
      // first keys (c <= c_ref) or when a probability of this chunk exceeds
      // 2^kMaxSlack.  Sum, accumulators and the partial's max all use the
      // same reference, so the result is exact in real arithmetic; a row
      // with no key keeps (-inf, 0, 0).
      float e[TILES][4];
#pragma unroll
      for (int t = 0; t < TILES; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) e[t][i] = fast_exp2(__builtin_fmaf(pr[t][i], smul, nm[nb]));
      bool exact = c <= c_ref;
      if (!exact) {
        // probabilities are >= 0 (or NaN), so their bit patterns order
        // as the values do; NaN lands above 2^kMaxSlack too
        uint32_t emax = __float_as_uint(e[0][0]);
#pragma unroll
        for (int t = 0; t < TILES; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) emax = max(emax, __float_as_uint(e[t][i]));
        exact = __builtin_amdgcn_ballot_w64(emax > __builtin_bit_cast(uint32_t, kSlackPow)) != 0;
      }
      if (exact) {
        float cmax = kNegInf;
#pragma unroll
        for (int t = 0; t < TILES; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) cmax = fmaxf(cmax, pr[t][i]);
        cmax = max4_rows(cmax);
        const float m_cand = fmaxf(m_run[nb], cmax * smul);
        float alpha = 1.0f;
        if (m_cand > m_run[nb] + kMaxSlack) {  // (a first key: -inf + slack is -inf)
          alpha = fast_exp2(m_run[nb] - m_cand);
          m_run[nb] = m_cand;
          nm[nb] = -m_cand;
#pragma unroll
          for (int t = 0; t < TILES; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              e[t][i] = fast_exp2(__builtin_fmaf(pr[t][i], smul, nm[nb]));
        }
        if (any_rescale(alpha)) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[nb][mt] *= alpha;
        }
        l_run[nb] *= alpha;
      }
      // the row sum adds the probabilities as P.V uses them (rounded to the
      // 16-bit type), two per packed dot
      float psum = l_run[nb];
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        pk[nb][2 * t] = pack2<DT>(e[t][0], e[t][1]);
        pk[nb][2 * t + 1] = pack2<DT>(e[t][2], e[t][3]);
        psum = add_pair<DT>(pk[nb][2 * t], psum);
        psum = add_pair<DT>(pk[nb][2 * t + 1], psum);
      }
      l_run[nb] = psum;
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      uint32_t vv[2 * TILES];
      vt_frag<D, TILES>(vb, mt, c16, j, vv);
#pragma unroll
      for (int nb = 0; nb < NR; ++nb) {
        if constexpr (TILES == 1) {
          acc[nb][mt] = mfma_k16<DT>(make_uint2(vv[0], vv[1]), make_uint2(pk[nb][0], pk[nb][1]),
                                     acc[nb][mt]);
        } else {
          // 32 keys (two tiles) per 16x16x32 product
#pragma unroll
          for (int tp = 0; tp < TILES / 2; ++tp)
            acc[nb][mt] = mfma_k32<DT>(
                make_uint4(vv[4 * tp], vv[4 * tp + 1], vv[4 * tp + 2], vv[4 * tp + 3]),
                make_uint4(pk[nb][4 * tp], pk[nb][4 * tp + 1], pk[nb][4 * tp + 2],
                           pk[nb][4 * tp + 3]),
                acc[nb][mt]);
        }
      }
    }
  };
  // The chunk loop, compiled once with and once without the soft-cap.
  auto walk = [&](auto capped_c) __attribute__((always_inline)) {
    if constexpr (kUnroll) {
#pragma clang loop unroll(disable)
      for (int c = c0; c <= c1; c += NBUF) {
        static_for<0, NBUF>([&](auto kc) __attribute__((always_inline)) {
          constexpr int k = decltype(kc)::value;
          if (k == 0 || c + k <= c1)
            chunk(c + k, buf(kc), buf(std::integral_constant<int, k + NBUF - 1>{}), capped_c);
        });
      }
    } else {
      int bi = 0;
#pragma clang loop unroll(disable)
      for (int c = c0; c <= c1; ++c) {
        chunk(c, lds_b0 + bi * 2 * CBYTES, lds_b0 + (bi == 0 ? NBUF - 1 : bi - 1) * 2 * CBYTES,
              capped_c);
        bi = bi == NBUF - 1 ? 0 : bi + 1;
      }
    }
  };
  if (p.cap_mul > 0.0f) walk(std::true_type{});
  else walk(std::false_type{});
  // the copies issued past the last chunk must land before the workgroup
  // (and its LDS) goes away
  __builtin_amdgcn_s_waitcnt(0);

  // ---- epilogue: each wavefront writes its own rows ----
#pragma unroll
  for (int nb = 0; nb < NR; ++nb) {
    const float l = sum4_rows(l_run[nb]);
    const int f = fw0 + 16 * nb + c16;
    if (f >= f_end || l == 0.0f) continue;  // past the end, or no key here
    const float inv = 1.0f / l;
    const int i = f / G;
    const int h = f - i * G;
    const int pos = L - n + i;
    const size_t row = (size_t)(q0 + i) * Hq + (size_t)g * G + h;
    if (key_lo(pos) / P == pos / P) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const size_t e = row * D + 16 * mt + 4 * j;
        const uint2 v = make_uint2(pack2<DT>(acc[nb][mt][0] * inv, acc[nb][mt][1] * inv),
                                   pack2<DT>(acc[nb][mt][2] * inv, acc[nb][mt][3] * inv));
        *reinterpret_cast<uint2*>(static_cast<char*>(p.out) + e * EB) = v;
      }
    } else {
      const size_t pi = row * p.num_parts + part;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        *reinterpret_cast<f32x4_t*>(p.tmp_out + pi * D + 16 * mt + 4 * j) = acc[nb][mt] * inv;
      if (j == 0) {
        p.max_logits[pi] = m_run[nb];
        p.exp_sums[pi] = l;
      }
    }
  }
}

}  // namespace pa
