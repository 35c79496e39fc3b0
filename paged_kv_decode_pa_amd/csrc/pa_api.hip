// C ABI of the library: argument checks, shape-dependent choices and kernel
// launches on the caller's stream.  Nothing here allocates, frees or
// synchronises.
#include <math.h>
#include <stdlib.h>

#include <atomic>

#include <hip/hip_runtime.h>

#include "../../include/pa.h"
#include "pa_launch.h"
#include "pa_plan.h"
#include "pa_reshape.h"

namespace {

// MI355X: 256 compute units.  Used only to size work, never for correctness.
constexpr int kNumCUs = 256;

// LDS bytes a multi-wavefront workgroup may take (of 160 KB per CU), so that
// at least two workgroups share a CU.
#ifndef PA_WG_LDS_CAP
#define PA_WG_LDS_CAP 65536
#endif

bool pow2_in(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

int ilog2(int v) {
  int r = 0;
  while ((1 << r) < v) ++r;
  return r;
}

bool supported_head_dim(int d) { return d == 64 || d == 128 || d == 256; }
bool valid_dtype(int dt) { return dt == PA_F32 || dt == PA_F16 || dt == PA_BF16; }
int elem_bytes(int dt) { return dt == PA_F32 ? 4 : 2; }

int num_parts(int max_context_len, int partition_size) {
  if (partition_size <= 0 || max_context_len <= 0) return 1;
  return (max_context_len + partition_size - 1) / partition_size;
}

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  if (!v || !*v) return dflt;
  return atoi(v);
}

// Workgroups one CU holds at once for a launch shape, from the runtime's
// occupancy calculator (query(&n) fills n), remembered in *slot; <= 0 when
// unknown.
template <typename Query>
int blocks_per_cu(std::atomic<int>* slot, Query&& query) {
  int v = slot->load(std::memory_order_relaxed);
  if (v == 0) {
    int n = 0;
    v = query(&n) && n > 0 ? n : -1;
    slot->store(v, std::memory_order_relaxed);
  }
  return v;
}

// Wavefronts per workgroup: enough to split a partition's chunks while each
// wavefront still streams several of them (four; a launch of fewer units
// than CUs is latency-bound, so there down to one each: the 4-sequence fp32
// workload's decode kernel 10.2 -> 6.6 us in rocprofv3 traces).
// PA_DECODE_WAVES overrides.
int waves_for(int tokens_per_part, int chunk_tokens, int units) {
  int forced = env_int("PA_DECODE_WAVES", 0);
  if (forced >= 1 && forced <= pa::kMaxWaves) return forced;
  int chunks = (tokens_per_part + chunk_tokens - 1) / chunk_tokens;
  const int per_wave = units < kNumCUs ? 1 : 4;
  int nw = 1;
  while (nw < pa::kMaxWaves && chunks >= 2 * per_wave * nw && units * nw < 8 * 4 * kNumCUs)
    nw *= 2;
  return nw;
}

int chunk_tokens(int dt, int D, int G) {
  const int epl = 16 / elem_bytes(dt);
  const int lpr = D / epl;
  const int rpi = 64 / lpr;
  const int ni = G >= 8 ? 4 : 8;
  return rpi * ni;
}

// LDS bytes one decode wavefront uses (DecodeShape::LDS_FLOATS).
size_t decode_lds_bytes(int dt, int D, int G) {
  const int slots = chunk_tokens(dt, D, G) * G;
  return sizeof(float) * (size_t)(slots + G + 64 + 2 * G + G * D);
}

}  // namespace

extern "C" {

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_EINVAL: return "invalid argument";
    case PA_EUNSUPPORTED: return "unsupported shape or dtype";
    case PA_EWORKSPACE: return "workspace missing or too small";
    case PA_ELAUNCH: return "kernel launch failed";
    case PA_ESCRATCH: return "the step needs more scratch than the static array holds";
    default: return "unknown status";
  }
}

int pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int num_tokens, int num_blocks,
                         int block_size, int num_kv_heads, int head_dim, pa_dtype dtype,
                         void* stream) {
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0) return PA_EINVAL;
  if (!valid_dtype(dtype) || !supported_head_dim(head_dim) || !pow2_in(block_size, 1, 256))
    return PA_EUNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PA_EINVAL;
  const int64_t row_bytes = (int64_t)num_kv_heads * head_dim * elem_bytes(dtype);
  const int row16 = (int)(row_bytes / 16);
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  hipStream_t s = static_cast<hipStream_t>(stream);
  pa::reshape_cache_kernel<<<dim3(num_tokens), dim3(256), 0, s>>>(
      static_cast<const uint4*>(key), static_cast<const uint4*>(value),
      static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), slot_mapping, num_slots, row16);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ELAUNCH;
}

int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping, int num_pairs,
                   int num_blocks, int block_size, int num_kv_heads, int head_dim,
                   pa_dtype dtype, void* stream) {
  if (num_pairs < 0 || num_blocks <= 0 || num_kv_heads <= 0) return PA_EINVAL;
  if (!valid_dtype(dtype) || !supported_head_dim(head_dim) || !pow2_in(block_size, 1, 256))
    return PA_EUNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_mapping) return PA_EINVAL;
  const int64_t block16 = (int64_t)block_size * num_kv_heads * head_dim * elem_bytes(dtype) / 16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  pa::copy_blocks_kernel<<<dim3(num_pairs), dim3(256), 0, s>>>(
      static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), block_mapping, num_blocks,
      block16);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ELAUNCH;
}

int pa_decode_partition_size(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                             int block_size, int max_context_len, int window, pa_dtype dtype) {
  (void)num_heads;
  (void)head_dim;
  (void)dtype;
  if (num_seqs <= 0 || num_kv_heads <= 0 || block_size <= 0 || max_context_len <= 0) return 0;
  int forced = env_int("PA_DECODE_PARTITION", -1);
  if (forced >= 0) return forced;
  const int span = window > 0 ? (window < max_context_len ? window : max_context_len)
                              : max_context_len;
  const long units = (long)num_seqs * num_kv_heads;
  // enough (sequence, head) units for the contexts' length: no split, so no
  // partials and no reduce launch (measured through pa_step: 64 sequences of
  // up to 1024 tokens x 4 heads, 37.6 us unsplit vs 39.4 us at 512-token
  // partitions, caches cold)
  if ((units >= kNumCUs && span <= 1024) || (units >= 4L * kNumCUs && span <= 2048)) return 0;
  int part = 512;
  if (part % block_size) part = block_size;
  return part;
}

// Workspace layout: the plan (sequence order [B] int32, item count, items
// [B*NP] int32 pairs, each padded to 256 bytes), then, when the keys are
// split, tmp_out [B,Hq,NP,D] f32, max_logits [B,Hq,NP] f32, exp_sums
// [B,Hq,NP] f32.
static size_t pad256(size_t n) { return (n + 255) & ~(size_t)255; }

static size_t plan_bytes(int num_seqs, int max_context_len, int partition_size) {
  const size_t np = (size_t)num_parts(max_context_len, partition_size);
  return pad256((size_t)num_seqs * 4) + 256 + pad256((size_t)num_seqs * np * 8);
}

static size_t partials_bytes(int num_seqs, int num_heads, int head_dim, int max_context_len,
                             int partition_size) {
  if (partition_size <= 0) return 0;
  const int np = num_parts(max_context_len, partition_size);
  if (np <= 1) return 0;
  const size_t rows = (size_t)num_seqs * num_heads * np;
  return rows * head_dim * sizeof(float) + 2 * rows * sizeof(float);
}

size_t pa_decode_workspace_size(int num_seqs, int num_heads, int head_dim, int max_context_len,
                                int partition_size) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || partition_size < 0) return 0;
  return plan_bytes(num_seqs, max_context_len, partition_size) +
         partials_bytes(num_seqs, num_heads, head_dim, max_context_len, partition_size);
}

// A checked pa_decode launch: the kernel parameters, the grid and whether
// the plan kernel must run first.
struct DecodeLaunch {
  pa::DecodeParams p;
  pa::Plan plan;
  bool need_plan, mfma, heads, loop, paged;
  int G, tiles, nw, head_dim;
  pa_dtype dtype;
  dim3 grid, block;
};

// Checks the arguments of pa_decode and makes its launch choices
// (*empty: nothing to launch).  Multi-query launches pass a table-row map
// (each query token runs as a sequence of its own; see pa_mq_attention).
static int decode_setup(void* out, void* workspace, size_t workspace_bytes, const void* q,
                        const void* k_cache, const void* v_cache, const int32_t* block_tables,
                        int max_blocks_per_seq, const int32_t* context_lens, int max_context_len,
                        int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                        int block_size, int num_blocks, float scale, float softcap, int window,
                        int partition_size, pa_dtype dtype, const int32_t* seq_row,
                        DecodeLaunch& dl, bool* empty) {
  *empty = true;
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || max_context_len < 0 || window < 0 || partition_size < 0)
    return PA_EINVAL;
  if (num_heads % num_kv_heads) return PA_EINVAL;
  if (!isfinite(scale) || !(softcap >= 0.0f) || !isfinite(softcap)) return PA_EINVAL;
  if (!valid_dtype(dtype) || !supported_head_dim(head_dim) || !pow2_in(block_size, 1, 256))
    return PA_EUNSUPPORTED;
  const int G = num_heads / num_kv_heads;
  // matrix cores take groups of 8 or 16 heads over 16-bit KV whose chunks
  // of 16 or 32 tokens fit in a page; PA_DECODE_MFMA=0 forces the vector path
  const bool mfma = (dtype == PA_F16 || dtype == PA_BF16) && (G == 8 || G == 16) &&
                    block_size >= 16 && env_int("PA_DECODE_MFMA", 1) != 0;
  if (!(G == 1 || G == 2 || G == 4 || G == 8 || (G == 16 && mfma))) return PA_EUNSUPPORTED;
  if (partition_size > 0 && partition_size % block_size) return PA_EINVAL;
  if ((long)max_context_len > (long)max_blocks_per_seq * block_size) return PA_EINVAL;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_EINVAL;
  *empty = false;

  const int np = num_parts(max_context_len, partition_size);
  const size_t need = pa_decode_workspace_size(num_seqs, num_heads, head_dim, max_context_len,
                                               partition_size);
  if (!workspace || workspace_bytes < need) return PA_EWORKSPACE;

  pa::DecodeParams p{};
  p.out = out;
  char* wsb = static_cast<char*>(workspace);
  pa::Plan plan;
  plan.order = reinterpret_cast<int32_t*>(wsb);
  plan.num_items = reinterpret_cast<int32_t*>(wsb + pad256((size_t)num_seqs * 4));
  plan.items = reinterpret_cast<int2*>(wsb + pad256((size_t)num_seqs * 4) + 256);
  p.order = plan.order;
  p.num_items = plan.num_items;
  p.items = plan.items;
  if (partials_bytes(num_seqs, num_heads, head_dim, max_context_len, partition_size)) {
    const size_t rows = (size_t)num_seqs * num_heads * np;
    float* ws = reinterpret_cast<float*>(wsb + plan_bytes(num_seqs, max_context_len,
                                                          partition_size));
    p.tmp_out = ws;
    p.max_logits = ws + rows * head_dim;
    p.exp_sums = p.max_logits + rows;
  }
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.seq_row = seq_row;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.max_context_len = max_context_len;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.num_blocks = num_blocks;
  p.log2_bs = ilog2(block_size);
  p.window = window;
  p.part = partition_size > 0 ? partition_size : (max_context_len > 0 ? max_context_len : 1);
  p.num_parts = np;
  if (softcap > 0.0f) {
    p.qk_mul = scale / softcap;
    p.cap_mul = softcap * pa::kLog2e;
  } else {
    p.qk_mul = scale * pa::kLog2e;
    p.cap_mul = 0.0f;
  }

  // two 16-token tiles per chunk when pages hold 32+ tokens and the K
  // fragments of both fit in registers (head_dim <= 128)
  const int tiles = block_size >= 32 && head_dim <= 128 ? 2 : 1;
  const int nt = mfma ? 16 * tiles : chunk_tokens(dtype, head_dim, G);
  const size_t lds_wave = mfma ? pa::decode_mfma_lds_bytes(head_dim, G, tiles)
                               : decode_lds_bytes(dtype, head_dim, G);
  const int span = window > 0 && window < p.part ? window : p.part;
  const long units = (long)num_seqs * num_kv_heads * np;
  // Matrix-core path: one wavefront per KV head in a workgroup, so the
  // heads' adjacent rows of a token are fetched together (PA_DECODE_HEADS=0
  // switches it off)
  const bool heads = mfma && num_kv_heads <= pa::kMaxWaves &&
                     (size_t)num_kv_heads * lds_wave <= PA_WG_LDS_CAP &&
                     env_int("PA_DECODE_HEADS", 1) != 0;
  int nw = heads ? num_kv_heads
                 : waves_for(span, nt, (int)(units < (1L << 30) ? units : (1L << 30)));
  while (!heads && nw > 1 && nw * lds_wave > PA_WG_LDS_CAP) nw /= 2;
  const long blocks = (long)num_seqs * (heads ? 1 : num_kv_heads) * np;
  if (blocks > 0x7fffffffL) return PA_EUNSUPPORTED;
  // Vector kernel: when the whole grid fits the chip at once as two-wavefront
  // workgroups, at least four per CU, over partitions of 32+ chunks, take
  // those, with wave priority from the chunks each wavefront has left, so
  // the workgroups sharing a CU finish together rather than oldest first
  // (sliding-window workload 53.1 -> 49.7 us, against eight-wavefront
  // workgroups; 128- to 512-token splits of the 64-sequence global layer,
  // with fewer workgroups or shorter partitions, lost 2-3 us to it).
  // PA_DECODE_PRIO sets the priority step (0: off); a forced
  // PA_DECODE_WAVES keeps its count.
  bool resident_pairs = false;
  if (!mfma && nw > 2 && env_int("PA_DECODE_WAVES", 0) == 0 && blocks >= 4L * kNumCUs &&
      span >= 32 * nt) {
    static std::atomic<int> occ_dec[3 * 3 * 4 * 2];
    const int paged_k = block_size >= nt;
    const int di = head_dim == 64 ? 0 : head_dim == 128 ? 1 : 2;
    const int gi = G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3;
    const int occ = blocks_per_cu(&occ_dec[((dtype * 3 + di) * 4 + gi) * 2 + paged_k], [&](int* n) {
      const dim3 blk(128);
      switch (dtype) {
        case PA_F32: return pa::launch_decode_f32(head_dim, G, paged_k, false, dim3(1), blk, nullptr, p, n);
        case PA_F16: return pa::launch_decode_f16(head_dim, G, paged_k, false, dim3(1), blk, nullptr, p, n);
        default: return pa::launch_decode_bf16(head_dim, G, paged_k, false, dim3(1), blk, nullptr, p, n);
      }
    });
    // (the grid of a split launch is rounded up to whole XCD rounds)
    const long grid2 = np > 1 ? (blocks + 8L * num_kv_heads - 1) / (8L * num_kv_heads) * 8L * num_kv_heads
                              : blocks;
    if (occ > 0 && grid2 <= (long)occ * kNumCUs) {
      nw = 2;
      resident_pairs = true;
    }
  }
  p.prio = mfma ? 0 : env_int("PA_DECODE_PRIO", resident_pairs ? 2 : 0);
  // One workgroup per (sequence, KV head, partition), unless that grid is
  // more than twice what the chip holds at once and spans many partitions:
  // workgroups are dispatched at a bounded rate, so a grid of mostly empty
  // partitions (one long sequence among short ones) would delay the real
  // work.  Then a smaller grid loops over the plan's list of non-empty
  // partitions.
  const long resident = (long)kNumCUs * 16 / nw;
  const bool loop = blocks > 2 * resident && np >= 8;
  if (!loop) plan.items = nullptr;
  // The longest-first order pays for its launch only over many sequences of
  // mixed length (measured: it gains 5% at 512 sequences and 4% at 64, and
  // costs 30% at 4 and 6% at 16); below 48 sequences the grid runs in input
  // order.  A looping launch always needs the plan's item list.
  // PA_DECODE_PLAN=0/1 overrides.
  // A grid that runs in one round (at most one workgroup per CU) has no
  // order to choose either.
  const int plan_env = env_int("PA_DECODE_PLAN", -1);
  const bool need_plan =
      loop || (plan_env >= 0 ? plan_env != 0 : num_seqs >= 48 && blocks > kNumCUs);
  if (!need_plan) p.order = nullptr;
  // XCD-grouped grid for per-head workgroups over split keys (measured: the
  // 16-sequence sliding-window workload 57 -> 52 us; the unsplit serving
  // batch loses 2.5 %, so it keeps the plain order).  PA_DECODE_XCD=0/1
  // overrides.
  long grid_blocks = loop ? 2 * resident : blocks;
  const int xcd_env = env_int("PA_DECODE_XCD", -1);
  const bool xcd = !loop && !heads && num_kv_heads > 1 &&
                   (xcd_env >= 0 ? xcd_env != 0 : np > 1);
  if (xcd) {
    const long units_bp = (long)num_seqs * np;
    p.xcd_units = (int)units_bp;
    const long per_round = 8L * num_kv_heads;
    grid_blocks = (blocks + per_round - 1) / per_round * per_round;
  }
  dl.p = p;
  dl.plan = plan;
  dl.need_plan = need_plan;
  dl.mfma = mfma;
  dl.heads = heads;
  dl.loop = loop;
  // chunks of nt tokens stay inside one page when block_size >= nt
  dl.paged = block_size >= nt;
  dl.G = G;
  dl.tiles = tiles;
  dl.nw = nw;
  dl.head_dim = head_dim;
  dl.dtype = dtype;
  dl.grid = dim3((unsigned)grid_blocks);
  dl.block = dim3(64 * nw);
  return PA_OK;
}

// Events pa_decode records around its decode kernel (pa_set_decode_events),
// per calling thread.
static thread_local hipEvent_t tl_decode_start = nullptr;
static thread_local hipEvent_t tl_decode_stop = nullptr;

// The decode kernel of a set-up launch (the plan, if needed, already queued).
static int decode_kernel_launch(const DecodeLaunch& dl, hipStream_t s) {
  const int D = dl.head_dim, G = dl.G;
  bool ok = false;
  if (dl.mfma) {
    ok = dl.dtype == PA_F16
             ? pa::launch_decode_mfma_f16(D, G, dl.tiles, dl.loop, dl.heads, dl.nw, dl.grid, s,
                                          dl.p)
             : pa::launch_decode_mfma_bf16(D, G, dl.tiles, dl.loop, dl.heads, dl.nw, dl.grid, s,
                                           dl.p);
  } else {
    switch (dl.dtype) {
      case PA_F32:
        ok = pa::launch_decode_f32(D, G, dl.paged, dl.loop, dl.grid, dl.block, s, dl.p);
        break;
      case PA_F16:
        ok = pa::launch_decode_f16(D, G, dl.paged, dl.loop, dl.grid, dl.block, s, dl.p);
        break;
      case PA_BF16:
        ok = pa::launch_decode_bf16(D, G, dl.paged, dl.loop, dl.grid, dl.block, s, dl.p);
        break;
    }
  }
  if (!ok) return PA_EUNSUPPORTED;
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ELAUNCH;
}

static int decode_impl(void* out, void* workspace, size_t workspace_bytes, const void* q,
                       const void* k_cache, const void* v_cache, const int32_t* block_tables,
                       int max_blocks_per_seq, const int32_t* context_lens, int max_context_len,
                       int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                       int num_blocks, float scale, float softcap, int window, int partition_size,
                       pa_dtype dtype, void* stream, const int32_t* seq_row) {
  DecodeLaunch dl;
  bool empty = true;
  const int st = decode_setup(out, workspace, workspace_bytes, q, k_cache, v_cache, block_tables,
                              max_blocks_per_seq, context_lens, max_context_len, num_seqs,
                              num_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                              softcap, window, partition_size, dtype, seq_row, dl, &empty);
  if (st != PA_OK || empty) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dl.need_plan)
    pa::plan_kernel<<<dim3(1), dim3(1024), 0, s>>>(context_lens, num_seqs, max_context_len,
                                                  window, dl.p.part, dl.plan);
  if (tl_decode_start && !seq_row && hipEventRecord(tl_decode_start, s) != hipSuccess)
    return PA_ELAUNCH;
  const int rc = decode_kernel_launch(dl, s);
  if (rc == PA_OK && tl_decode_stop && !seq_row && hipEventRecord(tl_decode_stop, s) != hipSuccess)
    return PA_ELAUNCH;
  return rc;
}

int pa_set_decode_events(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr)) return PA_EINVAL;
  tl_decode_start = static_cast<hipEvent_t>(start_event);
  tl_decode_stop = static_cast<hipEvent_t>(stop_event);
  return PA_OK;
}

int pa_decode(void* out, void* workspace, size_t workspace_bytes, const void* q,
              const void* k_cache, const void* v_cache, const int32_t* block_tables,
              int max_blocks_per_seq, const int32_t* context_lens, int max_context_len,
              int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
              int num_blocks, float scale, float softcap, int window, int partition_size,
              pa_dtype dtype, void* stream) {
  return decode_impl(out, workspace, workspace_bytes, q, k_cache, v_cache, block_tables,
                     max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, scale, softcap, window,
                     partition_size, dtype, stream, nullptr);
}

int pa_step(const pa_step_args* a, void* stream) {
  if (!a) return PA_EINVAL;
  const int T = a->num_tokens;
  if (T < 0) return PA_EINVAL;
  if (env_int("PA_STEP_FUSE", 1) == 0) {
    // the three entry points one after another
    int st = PA_OK;
    if (T > 0) {
      st = pa_reshape_and_cache(a->key, a->value, a->k_cache, a->v_cache, a->slot_mapping, T,
                                a->num_blocks, a->block_size, a->num_kv_heads, a->head_dim,
                                a->dtype, stream);
      if (st != PA_OK) return st;
    }
    st = pa_decode(a->out, a->workspace, a->workspace_bytes, a->q, a->k_cache, a->v_cache,
                   a->block_tables, a->max_blocks_per_seq, a->context_lens, a->max_context_len,
                   a->num_seqs, a->num_heads, a->num_kv_heads, a->head_dim, a->block_size,
                   a->num_blocks, a->scale, a->softcap, a->window, a->partition_size, a->dtype,
                   stream);
    if (st != PA_OK) return st;
    return pa_decode_reduce(a->out, a->workspace, a->workspace_bytes, a->context_lens,
                            a->max_context_len, a->num_seqs, a->num_heads, a->head_dim,
                            a->partition_size, a->window, a->dtype, stream);
  }
  if (T > 0) {  // the checks of pa_reshape_and_cache
    if (a->num_blocks <= 0 || a->num_kv_heads <= 0) return PA_EINVAL;
    if (!valid_dtype(a->dtype) || !supported_head_dim(a->head_dim) ||
        !pow2_in(a->block_size, 1, 256))
      return PA_EUNSUPPORTED;
    if (!a->key || !a->value || !a->k_cache || !a->v_cache || !a->slot_mapping) return PA_EINVAL;
  }
  DecodeLaunch dl;
  bool empty = true;
  int st = decode_setup(a->out, a->workspace, a->workspace_bytes, a->q, a->k_cache, a->v_cache,
                        a->block_tables, a->max_blocks_per_seq, a->context_lens,
                        a->max_context_len, a->num_seqs, a->num_heads, a->num_kv_heads,
                        a->head_dim, a->block_size, a->num_blocks, a->scale, a->softcap,
                        a->window, a->partition_size, a->dtype, nullptr, dl, &empty);
  if (st != PA_OK) return st;
  if (empty)
    return T > 0 ? pa_reshape_and_cache(a->key, a->value, a->k_cache, a->v_cache,
                                        a->slot_mapping, T, a->num_blocks, a->block_size,
                                        a->num_kv_heads, a->head_dim, a->dtype, stream)
                 : PA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Tail rows (one new token per sequence, at its last position): when
  // that is all the preparation launch would do (no plan), the vector decode
  // kernel writes them itself and the launch goes (global-layer workload,
  // 64 sequences: step 32.1 -> 29.8 us warm, 38.8 -> 35.0 us cold; with a
  // plan launch anyway, the serving batch lost 3 us to it).  PA_STEP_TAILS=0
  // switches it off.
  int T_prep = T;
  if (a->new_rows_at_tails && T > 0 && T == a->num_seqs && !dl.mfma && !dl.need_plan &&
      !dl.loop && env_int("PA_STEP_TAILS", 1) != 0) {
    dl.p.tail_k = a->key;
    dl.p.tail_v = a->value;
    dl.p.tail_slots = a->slot_mapping;
    T_prep = 0;
  }
  // One launch before the decode kernel: the new K/V rows and the plan.
  if (T_prep > 0 || dl.need_plan) {
    pa::PrepParams pp{};
    pp.context_lens = a->context_lens;
    pp.num_seqs = a->num_seqs;
    pp.max_context_len = a->max_context_len;
    pp.window = a->window;
    pp.part = dl.p.part;
    pp.plan = dl.plan;
    if (!dl.need_plan) pp.plan.order = nullptr;
    pp.key = static_cast<const uint4*>(a->key);
    pp.value = static_cast<const uint4*>(a->value);
    pp.k_cache = static_cast<uint4*>(a->k_cache);
    pp.v_cache = static_cast<uint4*>(a->v_cache);
    pp.slot_mapping = a->slot_mapping;
    pp.num_tokens = T_prep;
    pp.num_slots = (int64_t)a->num_blocks * a->block_size;
    pp.row16 = (int)((int64_t)a->num_kv_heads * a->head_dim * elem_bytes(a->dtype) / 16);
    const long blocks = 1 + ((long)T_prep + 3) / 4;
    if (blocks > 0x7fffffffL) return PA_EUNSUPPORTED;
    pa::step_prep_kernel<<<dim3((unsigned)blocks), dim3(1024), 0, s>>>(pp);
    if (hipGetLastError() != hipSuccess) return PA_ELAUNCH;
  }
  st = decode_kernel_launch(dl, s);
  if (st != PA_OK) return st;
  return pa_decode_reduce(a->out, a->workspace, a->workspace_bytes, a->context_lens,
                          a->max_context_len, a->num_seqs, a->num_heads, a->head_dim,
                          a->partition_size, a->window, a->dtype, stream);
}

int pa_decode_reduce(void* out, const void* workspace, size_t workspace_bytes,
                     const int32_t* context_lens, int max_context_len, int num_seqs,
                     int num_heads, int head_dim, int partition_size, int window,
                     pa_dtype dtype, void* stream) {
  if (num_seqs < 0 || num_heads <= 0 || max_context_len < 0 || window < 0 || partition_size < 0)
    return PA_EINVAL;
  if (!valid_dtype(dtype) || !supported_head_dim(head_dim)) return PA_EUNSUPPORTED;
  if (num_seqs == 0 ||
      partials_bytes(num_seqs, num_heads, head_dim, max_context_len, partition_size) == 0)
    return PA_OK;
  if (!out || !context_lens) return PA_EINVAL;
  const size_t need = pa_decode_workspace_size(num_seqs, num_heads, head_dim, max_context_len,
                                               partition_size);
  if (!workspace || workspace_bytes < need) return PA_EWORKSPACE;
  const int np = num_parts(max_context_len, partition_size);
  const size_t rows = (size_t)num_seqs * num_heads * np;
  const float* ws = reinterpret_cast<const float*>(
      static_cast<const char*>(workspace) + plan_bytes(num_seqs, max_context_len, partition_size));
  pa::ReduceParams p{};
  p.out = out;
  p.tmp_out = ws;
  p.max_logits = ws + rows * head_dim;
  p.exp_sums = p.max_logits + rows;
  p.context_lens = context_lens;
  p.max_context_len = max_context_len;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.window = window;
  p.part = partition_size;
  p.num_parts = np;
  const long groups = (long)num_seqs * num_heads;
  if (groups > 0x7fffffffL) return PA_EUNSUPPORTED;
  const dim3 grid((unsigned)groups), block(256);
  hipStream_t s = static_cast<hipStream_t>(stream);
#define PA_REDUCE_CASE(DTV, DT)                                                   \
  case DTV:                                                                       \
    if (head_dim == 64) pa::reduce_kernel<DT, 64><<<grid, block, 0, s>>>(p);      \
    else if (head_dim == 128) pa::reduce_kernel<DT, 128><<<grid, block, 0, s>>>(p); \
    else pa::reduce_kernel<DT, 256><<<grid, block, 0, s>>>(p);                   \
    break;
  switch (dtype) {
    PA_REDUCE_CASE(PA_F32, pa::DT_F32)
    PA_REDUCE_CASE(PA_F16, pa::DT_F16)
    PA_REDUCE_CASE(PA_BF16, pa::DT_BF16)
  }
#undef PA_REDUCE_CASE
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ELAUNCH;
}

// ---------------------------------------------------------------------------
// multi-query attention
// ---------------------------------------------------------------------------
// The tiled path takes 16-bit KV in pages of 16+ tokens; PA_MQ_TILED=0 forces
// the per-token path.
static bool mq_tiled(int dtype, int block_size, int max_query_len) {
  return (dtype == PA_F16 || dtype == PA_BF16) && block_size >= 16 && max_query_len > 1 &&
         env_int("PA_MQ_TILED", 1) != 0;
}

// 16-row blocks per wavefront: enough for a sequence's max_query_len * G
// rows, up to what the registers hold for the head size.
static int mq_row_blocks(int head_dim, int G, int max_query_len) {
  const int cap = head_dim == 64 ? 4 : head_dim == 128 ? 2 : 1;
  const long rows = (long)max_query_len * G;
  int nr = 1;
  while (nr < cap && 16L * nr < rows) nr *= 2;
  return nr;
}

// Row blocks per wavefront of the workgroup-shared kernel: two at head_dim
// 64 when a sequence has 256+ rows, else one, so that more workgroups stay
// resident (measured on the 4 x 2048-token prefill at head_dim 64: 138 us
// with two blocks against 147-149 with one; at head_dim 256 two blocks take
// the 512-token prompt chunk from 71 to 140 us).
static int mq_wg_row_blocks(int head_dim, int G, int max_query_len) {
  return head_dim == 64 && (long)max_query_len * G >= 256 ? 2 : 1;
}

// Tiles of R rows over every sequence's n * G rows: at most one partial tile
// per sequence, and never more tiles than rows.
static long mq_max_tiles(int num_seqs, int num_tokens, int G, int R) {
  const long rows = (long)num_tokens * G;
  const long t = rows / R + num_seqs;
  return t < rows ? t : rows;
}

// Workspace: vctx [T], vrow [T], tiles [max tiles at R = 16] int32 pairs,
// the tile and unit counts, (keys split) units [max tiles at R = 64 x NP]
// int32 pairs, then a decode workspace for T sequences.
static size_t mq_unit_cap(int num_seqs, int num_tokens, int G, int np) {
  return np > 1 ? (size_t)mq_max_tiles(num_seqs, num_tokens, G, 64) * np : 0;
}

static size_t mq_head_bytes(int num_seqs, int num_tokens, int G, int np) {
  return 2 * pad256((size_t)num_tokens * 4) +
         pad256((size_t)mq_max_tiles(num_seqs, num_tokens, G, 16) * 8) + 256 +
         pad256(mq_unit_cap(num_seqs, num_tokens, G, np) * 8);
}

int pa_mq_partition_size(int num_seqs, int num_tokens, int max_query_len, int num_heads,
                         int num_kv_heads, int head_dim, int block_size, int max_context_len,
                         int window, pa_dtype dtype) {
  if (num_seqs <= 0 || num_tokens <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads ||
      block_size <= 0 || max_context_len <= 0 || max_query_len <= 0)
    return 0;
  int forced = env_int("PA_DECODE_PARTITION", -1);
  if (forced >= 0) return forced;
  const int G = num_heads / num_kv_heads;
  long units;
  if (mq_tiled(dtype, block_size, max_query_len)) {
    int nr = mq_row_blocks(head_dim, G, max_query_len);
    const bool wg = (long)max_query_len * G > 16L * nr;
    if (wg) nr = mq_wg_row_blocks(head_dim, G, max_query_len);
    const int R = wg ? 64 * nr : 16 * nr;
    units = mq_max_tiles(num_seqs, num_tokens, G, R) * num_kv_heads;
  } else {
    units = (long)num_tokens * num_kv_heads;
  }
  const int span = window > 0 ? (window < max_context_len ? window : max_context_len)
                              : max_context_len;
  if (units >= 4L * kNumCUs && span <= 2048) return 0;
  int part = 512;
  if (part % block_size) part = block_size;
  return part;
}

size_t pa_mq_workspace_size(int num_seqs, int num_tokens, int num_heads, int num_kv_heads,
                            int head_dim, int max_context_len, int partition_size) {
  if (num_seqs <= 0 || num_tokens <= 0 || num_heads <= 0 || num_kv_heads <= 0 ||
      num_heads % num_kv_heads || head_dim <= 0 || partition_size < 0)
    return 0;
  return mq_head_bytes(num_seqs, num_tokens, num_heads / num_kv_heads,
                       num_parts(max_context_len, partition_size)) +
         pa_decode_workspace_size(num_tokens, num_heads, head_dim, max_context_len,
                                  partition_size);
}

// pa_mq_attention; with `rows`, its plan launch also writes the step's new
// K/V rows (the caller has checked them).
static int mq_attention_impl(void* out, void* workspace, size_t workspace_bytes, const void* q,
                             const int32_t* query_start, int num_tokens, int max_query_len,
                             const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, int max_blocks_per_seq,
                             const int32_t* context_lens, int max_context_len, int num_seqs,
                             int num_heads, int num_kv_heads, int head_dim, int block_size,
                             int num_blocks, float scale, float softcap, int window,
                             int partition_size, pa_dtype dtype, void* stream,
                             const pa::NewRows* rows) {
  if (num_seqs < 0 || num_tokens < 0 || num_heads <= 0 || num_kv_heads <= 0 ||
      num_blocks <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0 || window < 0 ||
      partition_size < 0)
    return PA_EINVAL;
  if (num_heads % num_kv_heads) return PA_EINVAL;
  if (num_tokens > 0 && (num_seqs == 0 || max_query_len < 1 || max_query_len > num_tokens))
    return PA_EINVAL;
  if (!isfinite(scale) || !(softcap >= 0.0f) || !isfinite(softcap)) return PA_EINVAL;
  if (!valid_dtype(dtype) || !supported_head_dim(head_dim) || !pow2_in(block_size, 1, 256))
    return PA_EUNSUPPORTED;
  if (partition_size > 0 && partition_size % block_size) return PA_EINVAL;
  if ((long)max_context_len > (long)max_blocks_per_seq * block_size) return PA_EINVAL;
  if (num_tokens == 0) return PA_OK;
  if (!out || !q || !query_start || !k_cache || !v_cache || !block_tables || !context_lens)
    return PA_EINVAL;
  const int G = num_heads / num_kv_heads;
  const bool tiled = mq_tiled(dtype, block_size, max_query_len);
  if (!tiled) {
    // the per-token path takes what the decode kernels take
    const bool mfma = (dtype == PA_F16 || dtype == PA_BF16) && (G == 8 || G == 16) &&
                      block_size >= 16 && env_int("PA_DECODE_MFMA", 1) != 0;
    if (!(G == 1 || G == 2 || G == 4 || G == 8 || (G == 16 && mfma))) return PA_EUNSUPPORTED;
  }
  const size_t need = pa_mq_workspace_size(num_seqs, num_tokens, num_heads, num_kv_heads,
                                           head_dim, max_context_len, partition_size);
  if (!workspace || workspace_bytes < need) return PA_EWORKSPACE;

  char* wsb = static_cast<char*>(workspace);
  int32_t* vctx = reinterpret_cast<int32_t*>(wsb);
  int32_t* vrow = reinterpret_cast<int32_t*>(wsb + pad256((size_t)num_tokens * 4));
  int2* tiles = reinterpret_cast<int2*>(wsb + 2 * pad256((size_t)num_tokens * 4));
  int32_t* num_tiles = reinterpret_cast<int32_t*>(
      wsb + 2 * pad256((size_t)num_tokens * 4) +
      pad256((size_t)mq_max_tiles(num_seqs, num_tokens, G, 16) * 8));
  const int np = num_parts(max_context_len, partition_size);
  int2* units = reinterpret_cast<int2*>(reinterpret_cast<char*>(num_tiles) + 256);
  const size_t head = mq_head_bytes(num_seqs, num_tokens, G, np);
  char* dws = wsb + head;
  const size_t dws_bytes = workspace_bytes - head;
  hipStream_t s = static_cast<hipStream_t>(stream);

  // More rows per (sequence, KV head) than one wavefront holds: the
  // workgroup-shared kernel (four wavefronts of rows over shared K/V chunks).
  // PA_MQ_WG=0/1 overrides.
  int nr = tiled ? mq_row_blocks(head_dim, G, max_query_len) : 1;
  const int nr_env = env_int("PA_MQ_NR", 0);
  if (tiled && (nr_env == 1 || nr_env == 2 || nr_env == 4)) nr = nr_env;
  const int wg_env = env_int("PA_MQ_WG", -1);
  const bool wg = tiled && (wg_env >= 0 ? wg_env != 0
                                        : (long)max_query_len * G > 16L * nr);
  if (wg && nr_env == 0) nr = mq_wg_row_blocks(head_dim, G, max_query_len);
  const int R = wg ? 64 * nr : 16 * nr;
  // keys split on the shared kernel: its grid walks the plan's sorted
  // (tile, partition) list (PA_MQ_UNITS=0: tiles in plan order, partitions
  // slowest)
  const bool by_units = wg && np > 1 && env_int("PA_MQ_UNITS", 1) != 0;
  const bool split = partials_bytes(num_tokens, num_heads, head_dim, max_context_len,
                                    partition_size) != 0;
  pa::MQPlanArgs pl{};
  pl.query_start = query_start;
  pl.context_lens = context_lens;
  pl.num_seqs = num_seqs;
  pl.num_tokens = num_tokens;
  pl.max_context_len = max_context_len;
  pl.window = window;
  pl.G = G;
  pl.R = R;
  pl.tiles = tiled ? tiles : nullptr;
  pl.tile_cap = (int)mq_max_tiles(num_seqs, num_tokens, G, R);
  pl.num_tiles = num_tiles;
  pl.part_size = partition_size;
  pl.units = by_units ? units : nullptr;
  pl.unit_cap = (int)mq_unit_cap(num_seqs, num_tokens, G, np);
  // token contexts: the per-token path's sequences, or the reduce's rows
  pl.vctx = !tiled || split ? vctx : nullptr;
  pl.vrow = tiled ? nullptr : vrow;
  if (rows != nullptr && rows->num_tokens > 0) {
    // copy workgroups: one 16-byte piece of K and of V per thread and pass,
    // at most two per CU
    const long pieces = (long)rows->num_tokens * rows->row16;
    const long need = (pieces + 1023) / 1024;
    const long wgs = need < 2L * kNumCUs ? need : 2L * kNumCUs;
    pa::mq_step_prep_kernel<<<dim3(1 + (unsigned)wgs), dim3(1024), 0, s>>>(pl, *rows);
  }
  else
    pa::mq_plan_kernel<<<dim3(1), dim3(1024), 0, s>>>(pl);
  if (hipGetLastError() != hipSuccess) return PA_ELAUNCH;

  int rc;
  if (!tiled) {
    // every query token is a decode sequence of context pos + 1
    rc = decode_impl(out, dws, dws_bytes, q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                     vctx, max_context_len, num_tokens, num_heads, num_kv_heads, head_dim,
                     block_size, num_blocks, scale, softcap, window, partition_size, dtype,
                     stream, vrow);
  } else {
    pa::MQParams p{};
    p.out = out;
    if (partials_bytes(num_tokens, num_heads, head_dim, max_context_len, partition_size)) {
      const size_t rows = (size_t)num_tokens * num_heads * np;
      float* ws = reinterpret_cast<float*>(dws + plan_bytes(num_tokens, max_context_len,
                                                            partition_size));
      p.tmp_out = ws;
      p.max_logits = ws + rows * head_dim;
      p.exp_sums = p.max_logits + rows;
    }
    p.tiles = tiles;
    p.num_tiles = num_tiles;
    p.units = by_units ? units : nullptr;
    p.q = q;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.query_start = query_start;
    p.max_blocks_per_seq = max_blocks_per_seq;
    p.max_context_len = max_context_len;
    p.num_heads = num_heads;
    p.num_kv_heads = num_kv_heads;
    p.group = G;
    p.num_blocks = num_blocks;
    p.log2_bs = ilog2(block_size);
    p.window = window;
    p.part = partition_size > 0 ? partition_size : (max_context_len > 0 ? max_context_len : 1);
    p.num_parts = np;
    if (softcap > 0.0f) {
      p.qk_mul = scale / softcap;
      p.cap_mul = softcap * pa::kLog2e;
    } else {
      p.qk_mul = scale * pa::kLog2e;
      p.cap_mul = 0.0f;
    }
    const long max_tiles = mq_max_tiles(num_seqs, num_tokens, G, R);
    p.max_tiles = (int)max_tiles;
    p.num_tokens = num_tokens;
    const long blocks = max_tiles * num_kv_heads * np;
    if (blocks > 0x7fffffffL) return PA_EUNSUPPORTED;
    const dim3 grid((unsigned)blocks);
    // per-wavefront kernel, keys not split: when the chip holds the whole
    // grid, tiles go to positions so that each CU's tiles pair long with
    // short (resident_tile; the shared kernel measured no better with it);
    // PA_MQ_RESIDENT=0 keeps the plan order
    const bool resident = np == 1 && env_int("PA_MQ_RESIDENT", 1) != 0;
    // wavefront priority by remaining chunks, in steps of 4 (measured on
    // the speculative-verification batch against steps of 1-12 and none);
    // PA_MQ_PRIO sets the step, 0 switches it off
    p.prio = env_int("PA_MQ_PRIO", 4);
    const int dti = dtype == PA_F16 ? 0 : 1;
    const int di = head_dim == 64 ? 0 : head_dim == 128 ? 1 : 2;
    auto set_resident = [&](int wgs_per_tile, int occ) {
      if (occ <= 0 || kNumCUs % wgs_per_tile) return;
      p.resident_period = kNumCUs / wgs_per_tile;
      p.resident_span = occ * p.resident_period;
    };
    bool ok;
    if (wg) {
      const int nbuf = env_int("PA_MQ_NBUF", 3);
      // head_dim 64 over 32-token pages: 64-key chunks (two pages, four
      // tiles) per workgroup step (PA_MQ_TILES=2 keeps one page a chunk)
      const int tiles_per_chunk =
          head_dim == 64 && block_size == 32 && nbuf == 3 && nr <= 2 &&
                  env_int("PA_MQ_TILES", 4) == 4
              ? 4
              : (block_size >= 32 && head_dim <= 128 ? 2 : 1);
      ok = dtype == PA_F16
               ? pa::launch_mq_wg_f16(head_dim, nr, tiles_per_chunk, nbuf, grid, s, p)
               : pa::launch_mq_wg_bf16(head_dim, nr, tiles_per_chunk, nbuf, grid, s, p);
    } else {
      const int tiles_per_chunk = block_size >= 32 && nr * head_dim <= 128 ? 2 : 1;
      // one wavefront per KV head when the heads' LDS fits two workgroups
      // per CU (PA_MQ_HEADS=0 switches it off)
      const size_t lds_heads = pa::mq_mfma_lds_bytes(head_dim, nr, tiles_per_chunk, true);
      const bool heads = num_kv_heads <= pa::kMaxWaves &&
                         (size_t)num_kv_heads * lds_heads <= 80 * 1024 &&
                         env_int("PA_MQ_HEADS", 1) != 0;
      const size_t lds_wave = pa::mq_mfma_lds_bytes(head_dim, nr, tiles_per_chunk, false);
      const int span = window > 0 && window < p.part ? window : p.part;
      int nw = heads ? num_kv_heads
                     : waves_for(span, 16 * tiles_per_chunk,
                                 (int)(blocks < (1L << 30) ? blocks : (1L << 30)));
      while (!heads && nw > 1 && nw * lds_wave > PA_WG_LDS_CAP) nw /= 2;
      const dim3 g_grid((unsigned)(heads ? blocks / num_kv_heads : blocks));
      if (resident) {
        static std::atomic<int> occ_mq[2 * 3 * 5 * 3 * 2 * 9];
        set_resident(heads ? 1 : num_kv_heads,
                     blocks_per_cu(
                         &occ_mq[((((dti * 3 + di) * 5 + nr) * 3 + tiles_per_chunk) * 2 + heads) *
                                     9 +
                                 nw],
                         [&](int* n) {
                           return dtype == PA_F16
                                      ? pa::launch_mq_mfma_f16(head_dim, nr, tiles_per_chunk,
                                                               heads, nw, g_grid, s, p, n)
                                      : pa::launch_mq_mfma_bf16(head_dim, nr, tiles_per_chunk,
                                                                heads, nw, g_grid, s, p, n);
                         }));
      }
      ok = dtype == PA_F16
               ? pa::launch_mq_mfma_f16(head_dim, nr, tiles_per_chunk, heads, nw, g_grid, s, p)
               : pa::launch_mq_mfma_bf16(head_dim, nr, tiles_per_chunk, heads, nw, g_grid, s, p);
    }
    if (!ok) return PA_EUNSUPPORTED;
    rc = hipGetLastError() == hipSuccess ? PA_OK : PA_ELAUNCH;
  }
  if (rc != PA_OK) return rc;
  // split-K partials of tokens whose keys span several partitions
  return pa_decode_reduce(out, dws, dws_bytes, vctx, max_context_len, num_tokens, num_heads,
                          head_dim, partition_size, window, dtype, stream);
}

int pa_mq_attention(void* out, void* workspace, size_t workspace_bytes, const void* q,
                    const int32_t* query_start, int num_tokens, int max_query_len,
                    const void* k_cache, const void* v_cache, const int32_t* block_tables,
                    int max_blocks_per_seq, const int32_t* context_lens, int max_context_len,
                    int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                    int num_blocks, float scale, float softcap, int window, int partition_size,
                    pa_dtype dtype, void* stream) {
  return mq_attention_impl(out, workspace, workspace_bytes, q, query_start, num_tokens,
                           max_query_len, k_cache, v_cache, block_tables, max_blocks_per_seq,
                           context_lens, max_context_len, num_seqs, num_heads, num_kv_heads,
                           head_dim, block_size, num_blocks, scale, softcap, window,
                           partition_size, dtype, stream, nullptr);
}

int pa_mq_step(const pa_mq_step_args* a, void* stream) {
  if (!a) return PA_EINVAL;
  const int T = a->num_new_rows;
  if (T < 0) return PA_EINVAL;
  if (T > 0) {  // the checks of pa_reshape_and_cache
    if (a->num_blocks <= 0 || a->num_kv_heads <= 0) return PA_EINVAL;
    if (!valid_dtype(a->dtype) || !supported_head_dim(a->head_dim) ||
        !pow2_in(a->block_size, 1, 256))
      return PA_EUNSUPPORTED;
    if (!a->key || !a->value || !a->k_cache || !a->v_cache || !a->slot_mapping) return PA_EINVAL;
  }
  if (T == 0 || a->num_tokens <= 0 || env_int("PA_STEP_FUSE", 1) == 0) {
    // the two entry points one after the other
    if (T > 0) {
      const int st = pa_reshape_and_cache(a->key, a->value, a->k_cache, a->v_cache,
                                          a->slot_mapping, T, a->num_blocks, a->block_size,
                                          a->num_kv_heads, a->head_dim, a->dtype, stream);
      if (st != PA_OK) return st;
    }
    return pa_mq_attention(a->out, a->workspace, a->workspace_bytes, a->q, a->query_start,
                           a->num_tokens, a->max_query_len, a->k_cache, a->v_cache,
                           a->block_tables, a->max_blocks_per_seq, a->context_lens,
                           a->max_context_len, a->num_seqs, a->num_heads, a->num_kv_heads,
                           a->head_dim, a->block_size, a->num_blocks, a->scale, a->softcap,
                           a->window, a->partition_size, a->dtype, stream);
  }
  pa::NewRows r{};
  r.key = static_cast<const uint4*>(a->key);
  r.value = static_cast<const uint4*>(a->value);
  r.k_cache = static_cast<uint4*>(a->k_cache);
  r.v_cache = static_cast<uint4*>(a->v_cache);
  r.slot_mapping = a->slot_mapping;
  r.num_tokens = T;
  r.num_slots = (int64_t)a->num_blocks * a->block_size;
  r.row16 = (int)((int64_t)a->num_kv_heads * a->head_dim * elem_bytes(a->dtype) / 16);
  return mq_attention_impl(a->out, a->workspace, a->workspace_bytes, a->q, a->query_start,
                           a->num_tokens, a->max_query_len, a->k_cache, a->v_cache,
                           a->block_tables, a->max_blocks_per_seq, a->context_lens,
                           a->max_context_len, a->num_seqs, a->num_heads, a->num_kv_heads,
                           a->head_dim, a->block_size, a->num_blocks, a->scale, a->softcap,
                           a->window, a->partition_size, a->dtype, stream, &r);
}

}  // extern "C"
