// Matrix-core decode kernel for large GQA groups (G = 8 or 16 query heads
// per KV head, f16/bf16): the group's q.k^T and P.V become dense 16x16
// tiles, so they run on MFMA instead of the vector ALUs.
//
// Per wavefront and chunk of NT = 16*TILES tokens (inside one KV page):
//   q.k^T   S^T[t][h] = K[t][:] . Q[h][:]   v_mfma_f32_16x16x32 (M = tokens,
//           N = heads, K = 32 dims per step).  The A operand is a K row slice:
//           lane (c16, j) holds token c16, dims 32s+8j..+8, a 16-byte load
//           straight from HBM; B is the query fragment (zero past head G).
//           The result leaves lane (c16, j) with head c16 at tokens
//           16t + 4j + i, i < 4.
//   softmax lane c16 owns query head c16: per-lane max/exp/sum, the group
//           max needs two xor shuffles (the 4 lanes of a head).
//   P.V     O^T[d][h] += V^T[d][t] . P^T[t][h]  (M = 16 dims, N = heads,
//           K = the chunk's tokens).  B = the lane's own probabilities, in
//           the token order the q.k result left them (any common order of
//           the K index is valid); A = V transposed, gathered from LDS.
//   The accumulators are rescaled only in chunks where some head's running
//   maximum moved.
//   PA_MFMA_DEPTH (2) chunks are in flight per wavefront: K in register
//   slots, V in LDS buffers.  V is copied HBM -> LDS by the buffer unit
//   (direct-to-LDS 16-byte loads, no registers in between).  Within a row the 16-byte segments are stored
//   XOR-swizzled (v_swz), so a transposed read hits distinct LDS banks.
#pragma once

#include "pa_kernels.h"

namespace pa {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

// 16x16x32 MFMA on 8 16-bit elements per lane (a and b as raw 16 bytes)
template <int DT>
__device__ __forceinline__ f32x4_t mfma_k32(const uint4& a, const uint4& b, f32x4_t c) {
  if constexpr (DT == DT_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// 16x16x16 MFMA on 4 16-bit elements per lane
template <int DT>
__device__ __forceinline__ f32x4_t mfma_k16(const uint2& a, const uint2& b, f32x4_t c) {
  if constexpr (DT == DT_F16)
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                     __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
}



// Chunks in flight per wavefront.  Measured on the long-context workload:
// 2 -> 153 us, 3 -> 160 us, 4 -> 175 us (each extra V buffer costs LDS and
// each K slot registers, and fewer wavefronts fit).
#ifndef PA_MFMA_DEPTH
#define PA_MFMA_DEPTH 2
#endif

template <int DT, int D, int G, int TILES>
struct MfmaShape {
  static constexpr int NT = 16 * TILES;             // tokens per chunk
  static constexpr int KS = D / 32;                 // q.k k-steps
  static constexpr int MT = D / 16;                 // P.V tiles over head_dim
  static constexpr int VBYTES = NT * D * 2;         // V chunk in LDS
  static constexpr int VLOADS = VBYTES / 1024;      // 1 KB direct-to-LDS loads
  static constexpr int DEPTH = PA_MFMA_DEPTH;       // chunks in flight per wavefront
  // LDS floats per wavefront: DEPTH V chunks, block-table window, max/sum,
  // and the accumulators staged for a merge -- in the V buffers when they
  // fit there (the merge comes after the last chunk's reads)
  static constexpr int V_F = DEPTH * VBYTES / 4;
  static constexpr int TBL = V_F;
  static constexpr int ML = TBL + 64;
  static constexpr bool ACC_IN_V = V_F >= G * (D + 4);
  static constexpr int ACC = ACC_IN_V ? 0 : ML + 2 * G;
  static constexpr int LDS_FLOATS = ACC_IN_V ? ML + 2 * G : ACC + G * (D + 4);
  static_assert(G == 8 || G == 16, "MFMA path: 8 or 16 query heads per KV head");
  static_assert(KS % 2 == 0, "k-steps come in pairs (whole-line K loads)");
  static_assert(VBYTES % 1024 == 0, "chunk must fill whole 1 KB LDS loads");
};

// byte offset of (row r, element d) of a V chunk in LDS: 16-byte segments
// XOR-swizzled by (r / 4) mod 4 (measured: a swizzle that also separates the
// four rows of one transposing read's lane group changes nothing)
template <int D>
__device__ __forceinline__ int v_swz(int r) { return ((r >> 2) & 3) << 1; }

template <int D>
__device__ __forceinline__ uint32_t v_lds_off(int r, int d) {
  return (uint32_t)(r * 2 * D + (((d >> 3) ^ v_swz<D>(r)) << 4) + ((d & 7) << 1));
}

// A operand of P.V for head-dim tile mt: lane (c16, j) gets V[16t + 4j +
// i][16mt + c16], i < 4, for each 16-token tile t, as 4 packed 16-bit values
// per tile, from the chunk in LDS by one transposing read per tile
// (ds_read_b64_tr_b16).  That read hands lane i of each 16-lane group
// element i % 4 of the 8 bytes at the address of lane 4e + i / 4, as its
// element e; so lane (c16, j) supplies the address of V row 16t + 4j +
// c16 / 4, dims 16mt + 4 (c16 % 4) .. + 3 (8 contiguous bytes: the swizzle
// moves whole 16-byte segments), and receives its column of the 4 x 16
// block of rows 16t + 4j .. + 3.
template <int D, int TILES>
__device__ __forceinline__ void vt_frag(const char* vb, int mt, int c16, int j,
                                        uint32_t (&vv)[2 * TILES]) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const int d = 16 * mt + 4 * (c16 & 3);
  // the swizzle depends on r mod 16 only: tile t's address is tile 0's
  // plus 16 t rows
  const char* a0 = vb + v_lds_off<D>(4 * j + (c16 >> 2), d);
#pragma unroll
  for (int t = 0; t < TILES; ++t) {
    const i16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(a0 + t * 16 * 2 * D));
    const uint2 u = __builtin_bit_cast(uint2, x);
    vv[2 * t] = u.x;
    vv[2 * t + 1] = u.y;
  }
}

// K fragments from whole 128-byte lines.  The A operand of q.k step s
// wants lane (c16, j) to hold token 16t + c16, dims 32s + 8j .. +8: a load
// shaped like that reads 64 bytes of each of 16 rows, half of each line
// (measured on this GPU: 5.8-6.0 TB/s for that pattern against 6.7-6.9 for
// whole lines).  Steps 2p and 2p + 1 cover line p of the rows, so their two
// loads are taken as whole lines instead, eight rows each:
//   load h (h = 0, 1) gives lane (c16, j) row 16t + 8h + c16 % 8, 16-byte
//   segment 8p + j + 4 (c16 / 8 xor h) of the head's row;
// kline_operands() then hands each lane its own row again.
__device__ __forceinline__ void kline_rowseg(int c16, int j, int t, int s, int& row, int& seg) {
  const int h = s & 1;
  row = 16 * t + 8 * h + (c16 & 7);
  seg = 8 * (s >> 1) + j + 4 * ((c16 >> 3) ^ h);
}

// The A operands of steps 2p (a0) and 2p + 1 (a1) from line p's two loads:
// lane (c16, j) needs row c16, segments 8p + j and 8p + 4 + j.  Lanes
// c16 < 8 find them in load 0, their own and that of lane c16 + 8; lanes
// c16 >= 8 in load 1, their own and that of lane c16 - 8: a select, and a
// select moved across the halves of each 16-lane row (DPP row rotate by 8).
__device__ __forceinline__ void kline_operands(int c16, const uint4& l0, const uint4& l1, uint4& a0,
                                               uint4& a1) {
  const bool hi8 = (c16 & 8) != 0;
  const uint4 x = hi8 ? l0 : l1;
  a0 = hi8 ? l1 : l0;
  a1.x = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x.x, 0x128, 0xF, 0xF, false);
  a1.y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x.y, 0x128, 0xF, 0xF, false);
  a1.z = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x.z, 0x128, 0xF, 0xF, false);
  a1.w = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x.w, 0x128, 0xF, 0xF, false);
}

// Max and sum over the four lanes c16 + 16 j' (j' < 4) that share a row of
// a 16x16 MFMA result, by the gfx950 lane-swap instructions: a permlane16
// swap of a value with itself leaves each lane its own value in one result
// and its xor-16 partner's in the other (rows of 16 lanes trade halves), a
// permlane32 swap likewise for the xor-32 partner.  Plain VALU moves, no
// LDS round trip.
__device__ __forceinline__ float max4_rows(float v) {
  const uint32_t x = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t y = __float_as_uint(v);
  const auto b = __builtin_amdgcn_permlane32_swap(y, y, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float sum4_rows(float v) {
  const uint32_t x = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t y = __float_as_uint(v);
  const auto b = __builtin_amdgcn_permlane32_swap(y, y, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// acc + lo + hi of two packed 16-bit values (one packed dot with (1, 1))
template <int DT>
__device__ __forceinline__ float add_pair(uint32_t pk, float acc) {
  if constexpr (DT == DT_F16)
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pk),
                                  f16x2_t{(_Float16)1.0f, (_Float16)1.0f}, acc, false);
  else
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk),
                                           bf16x2_t{(__bf16)1.0f, (__bf16)1.0f}, acc, false);
}

// true when any lane's alpha is below 1 (its running max moved): only then
// do the accumulators need rescaling
__device__ __forceinline__ bool any_rescale(float alpha) {
  return __builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0;
}

// Accumulators are staged in LDS as rows of D + 4 floats: 16-byte stores of
// 16 consecutive rows then fall in distinct bank groups.
template <int D>
constexpr int acc_stride() { return D + 4; }

// HEADS: one wavefront per KV head (the workgroup holds Hkv wavefronts and
// one (sequence, partition) unit for all heads), each walking every chunk of
// its head and writing its own rows; otherwise the workgroup's wavefronts
// split one head's chunks and merge in LDS.  A token's rows of all KV heads
// are adjacent in memory: with HEADS they are fetched by one workgroup (one
// XCD) at about the same time.
template <int DT, int D, int G, int TILES, bool LOOP, bool HEADS = false>
__global__ __launch_bounds__(64 * kMaxWaves) void decode_mfma_kernel(DecodeParams p) {
  using S = MfmaShape<DT, D, G, TILES>;
  constexpr int NT = S::NT, KS = S::KS, MT = S::MT, VLOADS = S::VLOADS;
  constexpr int EB = 2;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int c16 = lane & 15;
  const int j = lane >> 4;

  extern __shared__ __align__(16) float smem[];
  float* s_wave = smem + w * S::LDS_FLOATS;
  char* vbuf = reinterpret_cast<char*>(s_wave);
  int32_t* tbl = reinterpret_cast<int32_t*>(s_wave + S::TBL);

  // the chunks of a unit this wavefront takes: w, w + nw, ... (all of them
  // with HEADS)
  const int cw = HEADS ? 0 : w;
  const int cstride = HEADS ? 1 : nw;

  for_units<DT, D, G, LOOP, HEADS>(p, [&](const Unit& u) {
  const int Hq = p.num_heads;
  const int b = u.b, g = u.g, lo = u.lo, hi = u.hi;

  // query fragments (B operand of q.k): head c16, dims 32s + 8j .. +8
  uint4 qf[KS];
  {
    const char* qb = static_cast<const char*>(p.q) +
                     (((size_t)b * Hq + (size_t)g * G + c16) * D + 8 * j) * EB;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[s] = c16 < G ? ld16(qb + (size_t)s * 32 * EB) : make_uint4(0, 0, 0, 0);
  }

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

  const uint32_t row_bytes = (uint32_t)(p.num_kv_heads * D * EB);
  const uint32_t page_bytes = row_bytes << log2_bs;
  const uint32_t head_bytes = (uint32_t)(g * D * EB);
  const char* kbase = static_cast<const char*>(p.k_cache);
  const char* vbase = static_cast<const char*>(p.v_cache);
  const char* dummy = static_cast<const char*>(p.q) + ((size_t)b * Hq + (size_t)g * G) * D * EB;

  // per-lane constants of the V copy: instruction i moves LDS bytes
  // [1024 i, 1024 i + 1024); lane l's 16 bytes hold row r, stored segment
  // sg ^ f(r) of global segment sg
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
    int rlo, rhi;  // clamp bounds of chunk rows
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

  float m_run = kNegInf;  // running max (base 2) of query head c16
  float l_run = 0.0f;     // this lane's share of its running sum
  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  const int c0 = lo / NT;
  const int c1 = (hi - 1) / NT;
  constexpr int NK = TILES * KS;  // K loads per chunk
  constexpr int NV = VLOADS;      // V copies per chunk
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

  // One chunk cc: q.k on the K slot, then that slot and V buffer `vb` are
  // refilled with chunk cn (a few bytes of q past the last chunk), so DEPTH
  // chunks stay in flight while this one is computed.  A chunk past the end
  // is fully masked and leaves the running state unchanged.
  auto step = [&](int cc, int cn, uint4 (&k)[TILES][KS], char* vb) __attribute__((always_inline)) {
    f32x4_t sc[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      sc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < KS; s += 2) {
        uint4 a0, a1;
        kline_operands(c16, k[t][s], k[t][s + 1], a0, a1);
        sc[t] = mfma_k32<DT>(a0, qf[s], sc[t]);
        sc[t] = mfma_k32<DT>(a1, qf[s + 1], sc[t]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    Addr an;
    addr_of(cn, an);
    issue_k(an, k);
    __builtin_amdgcn_sched_barrier(0);

    // online softmax for head c16 over tokens 16t + 4j + i
    const int cs = cc * NT;
    float pr[TILES][4];
    float cmax = kNegInf;
    if (p.cap_mul > 0.0f) {
#pragma unroll
      for (int t = 0; t < TILES; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[t][i] = p.cap_mul * tanh_def(sc[t][i] * p.qk_mul);
    } else {
#pragma unroll
      for (int t = 0; t < TILES; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[t][i] = sc[t][i] * p.qk_mul;
    }
    if (cs < lo || cs + NT > hi) {  // only a unit's first and last chunks need the mask
#pragma unroll
      for (int t = 0; t < TILES; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pos = cs + 16 * t + 4 * j + i;
          pr[t][i] = (pos >= lo && pos < hi) ? pr[t][i] : kNegInf;
        }
    }
#pragma unroll
    for (int t = 0; t < TILES; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) cmax = fmaxf(cmax, pr[t][i]);
    cmax = max4_rows(cmax);
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = fast_exp2(m_run - m_new);
    float psum = 0.0f;
#pragma unroll
    for (int t = 0; t < TILES; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[t][i] = fast_exp2(pr[t][i] - m_new);
        psum += pr[t][i];
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (any_rescale(alpha)) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] *= alpha;
    }

    // P^T fragment: this lane's probabilities in (tile, i) order
    uint32_t pk[2 * TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      pk[2 * t] = pack2<DT>(pr[t][0], pr[t][1]);
      pk[2 * t + 1] = pack2<DT>(pr[t][2], pr[t][3]);
    }

    // O^T += V^T . P^T, V^T gathered from LDS in the same token order.
    // Issued after this chunk's V copy: the other slot's K and V, and the K
    // just issued.
    __builtin_amdgcn_s_waitcnt(vmcnt_only((S::DEPTH - 1) * (NK + NV) + NK));
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      uint32_t vv[2 * TILES];
      vt_frag<D, TILES>(vb, mt, c16, j, vv);
      if constexpr (TILES == 2)
        acc[mt] = mfma_k32<DT>(make_uint4(vv[0], vv[1], vv[2], vv[3]),
                               make_uint4(pk[0], pk[1], pk[2], pk[3]), acc[mt]);
      else
        acc[mt] = mfma_k16<DT>(make_uint2(vv[0], vv[1]), make_uint2(pk[0], pk[1]), acc[mt]);
    }
    // refill the buffer once every lane has read it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    __builtin_amdgcn_sched_barrier(0);
    vcopy(an, vb);
    __builtin_amdgcn_sched_barrier(0);
  };

  constexpr int DEPTH = S::DEPTH;
  uint4 kf[DEPTH][TILES][KS];
  int c = c0 + cw;
  if (c <= c1) {
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) {
      Addr a;
      addr_of(c + i * cstride, a);
      issue_k(a, kf[i]);
      __builtin_amdgcn_sched_barrier(0);
      vcopy(a, vbuf + i * S::VBYTES);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (DEPTH == 2) {
      // the two V buffers as restrict pointers: the compiler's own wait
      // before one buffer's LDS reads then leaves the other buffer's copy in
      // flight (the explicit wait in step covers what the reads need)
      auto two = [&](char* __restrict__ b0, char* __restrict__ b1) __attribute__((always_inline)) {
        step(c, c + 2 * cstride, kf[0], b0);
        step(c + cstride, c + 3 * cstride, kf[1], b1);
      };
#pragma clang loop unroll(disable)
      for (; c <= c1; c += 2 * cstride) two(vbuf, vbuf + S::VBYTES);
    } else {
#pragma clang loop unroll(disable)
      for (; c <= c1; c += DEPTH * cstride) {
#pragma unroll
        for (int i = 0; i < DEPTH; ++i)
          step(c + i * cstride, c + (i + DEPTH) * cstride, kf[i], vbuf + i * S::VBYTES);
      }
    }
  }
  // drain the trailing loads before the wavefront moves on
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();

  if constexpr (HEADS) {
    // this wavefront holds its head's whole unit: write from registers
    const float l = sum4_rows(l_run);
    if (c16 < G) {
      const float inv = 1.0f / l;
      const size_t row = (size_t)b * Hq + (size_t)g * G + c16;
      if (u.single) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const uint2 v = make_uint2(pack2<DT>(acc[mt][0] * inv, acc[mt][1] * inv),
                                     pack2<DT>(acc[mt][2] * inv, acc[mt][3] * inv));
          *reinterpret_cast<uint2*>(static_cast<char*>(p.out) + (row * D + 16 * mt + 4 * j) * EB) =
              v;
        }
      } else {
        const size_t pi = row * p.num_parts + u.part;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          *reinterpret_cast<f32x4_t*>(p.tmp_out + pi * D + 16 * mt + 4 * j) = acc[mt] * inv;
        if (j == 0) {
          p.max_logits[pi] = m_run;
          p.exp_sums[pi] = l;
        }
      }
    }
    return;
  }

  // ---- epilogue: sums over the head's four lanes, then the LDS merge ----
  l_run = sum4_rows(l_run);
  if (c16 < G) {
    if (j == 0) {
      s_wave[S::ML + c16] = m_run;
      s_wave[S::ML + G + c16] = l_run;
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      *reinterpret_cast<f32x4_t*>(s_wave + S::ACC + c16 * acc_stride<D>() + 16 * mt + 4 * j) =
          acc[mt];
  }
  __syncthreads();
  merge_store<DT, D, G>(p, u, smem, S::LDS_FLOATS, S::ML, S::ACC, nw, acc_stride<D>());
  });
}

}  // namespace pa
