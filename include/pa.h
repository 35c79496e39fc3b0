/*
 * pa.h - paged KV-cache decode attention for AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  Every pointer argument is a DEVICE
 * pointer owned by the caller unless stated otherwise; the library never
 * allocates, frees or synchronises on these calls.  Work is enqueued on the
 * caller's HIP stream (`stream` is a hipStream_t; NULL means the default
 * stream) and calls on one stream run in order:
 *     pa_reshape_and_cache -> pa_decode -> pa_decode_reduce.
 *
 * What is computed.  A paged KV cache holds keys and values in fixed-size
 * physical blocks; a per-sequence block table maps logical block j of
 * sequence b to physical block block_tables[b][j], and token t of the
 * sequence lives at slot t % block_size of that block (ovshake/nano-vllm
 * README, "Key Concepts Explained: PagedAttention"; flex-nano-vllm README,
 * file list: page table and paged kv cache).  In the decode phase each
 * sequence contributes one new token (same README, "Key Concepts Explained:
 * KV Cache"), whose query attends to the sequence's cached keys:
 *     s_t = scale * q . k_t                      (X-Ray Mode, Step 2)
 *     s_t = softcap * tanh(s_t / softcap)        if softcap > 0
 *     out = sum_t softmax(s)_t v_t   over t in [max(0, L - window), L)
 * Query head h reads KV head floor(h / G), G = num_heads / num_kv_heads
 * (grouped-query attention; X-Ray Mode, Step 1 GQA note).  The soft-cap and
 * the window follow the public Gemma-2 attention definition (the pages name
 * Gemma 2 but print neither rule).
 *
 * Layouts (row-major, innermost last):
 *   q, out          [num_seqs, num_heads, head_dim]               dtype
 *   key, value      [num_tokens, num_kv_heads, head_dim]          dtype
 *   k_cache,v_cache [num_blocks, block_size, num_kv_heads, head_dim] dtype
 *   block_tables    [num_seqs, max_blocks_per_seq] int32 physical ids
 *   context_lens    [num_seqs] int32: tokens in the sequence, counting the
 *                   new one (whose K/V reshape_and_cache has written)
 *   slot_mapping    [num_tokens] int64: physical_block*block_size + offset,
 *                   or -1 to skip the token
 *
 * Errors.  Every call returns PA_OK (0) or a negative pa_status.  All checks
 * on host-visible arguments run before anything is enqueued, so a failed call
 * leaves every buffer untouched.  Device-resident contents are the caller's
 * contract and are not checked on the host: block ids referenced by the first
 * ceil(L/block_size) table entries lie in [0, num_blocks), context_lens[b] <=
 * max_context_len, and slot_mapping holds no duplicate slot.  The kernels
 * clamp out-of-range ids and lengths so that a broken contract gives wrong
 * numbers rather than an out-of-bounds access.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 } pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_EINVAL = -1,        /* bad pointer, size or value                      */
  PA_EUNSUPPORTED = -2,  /* valid but not built: dtype, head_dim, group size */
  PA_EWORKSPACE = -3,    /* workspace missing or smaller than required      */
  PA_ELAUNCH = -4,       /* the HIP runtime refused the launch              */
  PA_ESCRATCH = -5       /* pa_step_static: the step needs more scratch than
                            PA_STATIC_SCRATCH_BYTES                         */
} pa_status;

/* Text for a status code (static storage, never NULL). */
const char* pa_status_string(int status);

/*
 * Write the K/V rows of new tokens into their physical slots:
 *   k_cache.flat[slot_mapping[i]] = key[i], v_cache.flat[...] = value[i]
 * with flat = view [num_blocks*block_size, num_kv_heads, head_dim].  With a
 * KV cache, a step computes K and V for its new tokens only and appends them
 * to what is cached (ovshake/nano-vllm README, "Key Concepts Explained: KV
 * Cache"); the cache is the block pool of the same section's PagedAttention
 * figure, so a token's slot is physical_block * block_size + offset.  Rows
 * with slot -1 are skipped; slots outside the pool (negative, or >=
 * num_blocks * block_size) are skipped as well, leaving the caches untouched.
 * The copy is bit-exact (NaN payloads included).  Other slots are not
 * touched.  key, value and slot_mapping are read only; k_cache and v_cache
 * are written in place.  Errors: PA_EINVAL for a negative num_tokens, a
 * non-positive pool size or head count, or a null pointer when num_tokens >
 * 0; PA_EUNSUPPORTED for the shapes below; PA_ELAUNCH if the launch fails.
 * Supported: dtype any; head_dim in {64,128,256}; block_size a power of two
 * in [1,256]; num_tokens >= 0 (0 is a no-op).
 */
int pa_reshape_and_cache(const void* key, const void* value,
                         void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int num_tokens,
                         int num_blocks, int block_size, int num_kv_heads,
                         int head_dim, pa_dtype dtype, void* stream);

/*
 * Copy whole KV blocks (every slot, every KV head, K and V):
 *   k_cache[dst] = k_cache[src], v_cache[dst] = v_cache[src]
 * for each pair (src, dst) = (block_mapping[2i], block_mapping[2i+1]),
 * i < num_pairs.  This is the copy-on-write step of block sharing: sequences
 * with a common prefix point their block tables at the same physical blocks
 * (ovshake/nano-vllm README, "Features": prefix caching shares KV blocks of
 * common prefixes; GeeeekExplorer/nano-vllm, "Features": non-contiguous
 * blocks enable sharing), and a sequence about to write into a shared,
 * partly filled block first gets a private copy.  Bit-exact.  Pairs with an
 * id outside [0, num_blocks) are skipped.  Caller contract: no block is the
 * destination of two pairs or both a source and a destination.
 *   block_mapping  [num_pairs, 2] int64, device memory
 */
int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping, int num_pairs,
                   int num_blocks, int block_size, int num_kv_heads, int head_dim,
                   pa_dtype dtype, void* stream);

/*
 * The partition size the library would pick for this shape (tokens per
 * split-K partition; 0 means one partition per sequence).  A partition is
 * one block of the blocked, numerically stable attention the pages describe
 * for flash attention (sourcepulse MinivLLM summary, "How It Works"): each
 * is attended on its own and the blocks are merged by pa_decode_reduce.
 * Host-only; returns 0 for non-positive sizes.
 */
int pa_decode_partition_size(int num_seqs, int num_heads, int num_kv_heads,
                             int head_dim, int block_size, int max_context_len,
                             int window, pa_dtype dtype);

/*
 * Bytes of workspace pa_decode needs (0 only when num_seqs <= 0).  It holds
 * the work order and, when keys are split into partitions (the blocks of
 * blocked attention: sourcepulse MinivLLM summary, "How It Works"), each
 * block's partial result -- its running maximum, its sum of exponentials and
 * its normalised output -- for pa_decode_reduce to merge.  The caller
 * allocates it in device memory and passes it to pa_decode and
 * pa_decode_reduce; its contents need no initialisation.  Host-only;
 * returns 0 for invalid sizes.  Layout:
 *   order      [num_seqs] int32, padded to 256 bytes: the sequences sorted
 *              longest first, written by pa_decode itself
 *   count      one int32, padded to 256 bytes, and
 *   items      [num_seqs * NP] int32 pairs, padded to 256 bytes: the
 *              non-empty (sequence, partition) list of a looping launch
 * and, when the keys are split (partition_size > 0 and NP > 1), after them:
 *   tmp_out    [num_seqs, num_heads, NP, head_dim] float32
 *   max_logits [num_seqs, num_heads, NP]           float32 (base-2 logits)
 *   exp_sums   [num_seqs, num_heads, NP]           float32
 * with NP = ceil(max_context_len / partition_size).  Host-only.
 */
size_t pa_decode_workspace_size(int num_seqs, int num_heads, int head_dim,
                                int max_context_len, int partition_size);

/*
 * Decode attention, first pass.  The keys of each sequence are split at
 * absolute positions that are multiples of partition_size (0 = one partition
 * per sequence).  The workspace (pa_decode_workspace_size bytes) is
 * required; its contents need no initialisation and are overwritten.  A
 * sequence whose attended keys fall in a single partition gets its output
 * written to `out` directly; for the others each partition
 * writes normalised partial outputs plus its running max and sum to the
 * workspace, and pa_decode_reduce must follow on the same stream.
 * An empty sequence (context_lens[b] == 0) gets out = 0.
 *   scale          multiplies q . k (e.g. 1/sqrt(head_dim))
 *   softcap        > 0: logits capped to softcap*tanh(s/softcap); 0: off
 *   window         > 0: attend to the last `window` keys only; 0: off
 *   max_context_len  host-side upper bound of context_lens (sizes the grid);
 *                  must be <= max_blocks_per_seq * block_size
 *   partition_size 0, or a positive multiple of block_size
 * Supported: num_heads/num_kv_heads in {1,2,4,8}; head_dim in {64,128,256};
 * block_size a power of two in [1,256]; dtype f32, f16, bf16 (q, caches and
 * out share it; arithmetic is float32).
 */
int pa_decode(void* out, void* workspace, size_t workspace_bytes,
              const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, int max_blocks_per_seq,
              const int32_t* context_lens, int max_context_len,
              int num_seqs, int num_heads, int num_kv_heads, int head_dim,
              int block_size, int num_blocks, float scale, float softcap,
              int window, int partition_size, pa_dtype dtype, void* stream);

/*
 * Measurement hook: while set, every pa_decode call made by this thread
 * records `start_event` on its stream right before its decode kernel and
 * `stop_event` right after it (two hipEvent_t created by the caller), so
 * the pair brackets that one kernel -- not the plan launch before it.
 * pa_decode returns PA_ELAUNCH if a record fails.  (NULL, NULL) clears the
 * hook; one NULL alone is PA_EINVAL.  The library never creates or frees
 * the events.
 */
int pa_set_decode_events(void* start_event, void* stop_event);

/*
 * Measurement aid, not part of the attention path: one streaming pass that
 * reads `bytes` of device memory at `buf` (16-byte aligned, a multiple of
 * 16 bytes) with `grid` workgroups of 256 threads, 16-byte non-temporal
 * loads, eight in flight per thread, each workgroup step one contiguous
 * 32 KB block, the blocks dealt to the workgroups in turn.  It gives the
 * read bandwidth a plain
 * kernel reaches on this GPU: the practical ceiling the memory-bound
 * decode kernels are reported against next to the data sheet's peak.
 * `sink` is a 4-byte device word the kernel may write (it practically never
 * does).  Nothing is allocated; the launch is queued on `stream`.  Returns
 * PA_EINVAL for bad arguments, PA_ELAUNCH if the launch fails.
 */
int pa_read_bandwidth_probe(const void* buf, size_t bytes, int grid, void* sink, void* stream);

/*
 * Decode attention, reduce pass: for each sequence with more than one
 * non-empty partition, combine the partials with weights
 * exp_sum_p * 2^(max_logit_p - max_p' max_logit_p') and write `out`.  This
 * is the merge step of blocked, numerically stable attention (sourcepulse
 * MinivLLM summary, "How It Works": attention computed block by block): each
 * block's result is rescaled to the common maximum before the sums are
 * combined, so the output equals softmax attention over all the keys.
 * Sequences handled by pa_decode alone are left as they are.  A no-op when
 * partition_size is 0.  Arguments must match the pa_decode call;
 * `workspace` is the one pa_decode wrote (read only here) and
 * `workspace_bytes` its size, checked against pa_decode_workspace_size
 * (PA_EWORKSPACE when null or smaller).  `out` is written for merged sequences only.
 * Errors: PA_EINVAL for negative sizes or null pointers, PA_EUNSUPPORTED
 * for an unsupported dtype or head_dim, PA_ELAUNCH if the launch fails.
 */
int pa_decode_reduce(void* out, const void* workspace, size_t workspace_bytes,
                     const int32_t* context_lens, int max_context_len,
                     int num_seqs, int num_heads, int head_dim,
                     int partition_size, int window, pa_dtype dtype,
                     void* stream);

/*
 * Multi-query attention: a sequence brings n_b >= 0 new tokens at once, the
 * last n_b of its context_lens[b] positions (a prompt chunk under chunked
 * prefill, or the draft tokens a speculative-decoding step verifies:
 * ovshake/nano-vllm README, "Features", "Advanced Scheduling" and
 * "Optimizations").  Attention is causal (the self-attention chapter under
 * that README's "Educational Modes"): the new token at position
 * pos = L_b - n_b + i attends to the keys at [max(0, pos+1-window), pos]
 * (window 0: [0, pos]) with the decode rule above, so n_b = 1 is decode and
 * n_b = L_b is the prefill of a whole prompt.  Every new token's K/V row must
 * already be in the cache (pa_reshape_and_cache first).  One call enqueues
 * the plan, the attention pass and, when keys are split, the reduce.
 *   q, out        [num_tokens, num_heads, head_dim], tokens packed sequence
 *                 by sequence in position order
 *   query_start   [num_seqs + 1] int32: sequence b owns rows
 *                 query_start[b] .. query_start[b+1]-1; query_start[0] = 0,
 *                 non-decreasing, query_start[num_seqs] = num_tokens
 *   context_lens  [num_seqs] int32, counting all new tokens (n_b <= L_b)
 *   max_query_len host-side hint >= 1 (the largest n_b); it picks the tile
 *                 shape only, results do not depend on it
 *   partition_size  0, or a positive multiple of block_size
 * The query_start contract and n_b <= L_b <= max_context_len are device-side
 * contracts (not checked).  Supported: as pa_decode, and any group size
 * for f16/bf16 with block_size >= 16 (matrix-core path; other shapes run
 * each token through the decode kernels).
 */
int pa_mq_partition_size(int num_seqs, int num_tokens, int max_query_len, int num_heads,
                         int num_kv_heads, int head_dim, int block_size, int max_context_len,
                         int window, pa_dtype dtype);

/* Bytes of workspace pa_mq_attention needs (0 when num_tokens <= 0). */
size_t pa_mq_workspace_size(int num_seqs, int num_tokens, int num_heads, int num_kv_heads,
                            int head_dim, int max_context_len, int partition_size);

int pa_mq_attention(void* out, void* workspace, size_t workspace_bytes, const void* q,
                    const int32_t* query_start, int num_tokens, int max_query_len,
                    const void* k_cache, const void* v_cache, const int32_t* block_tables,
                    int max_blocks_per_seq, const int32_t* context_lens, int max_context_len,
                    int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                    int num_blocks, float scale, float softcap, int window, int partition_size,
                    pa_dtype dtype, void* stream);

/*
 * One multi-query layer-step: the new tokens' K and V are appended to the
 * cache and the new tokens attend (ovshake/nano-vllm README, "Key Concepts
 * Explained: KV Cache": a step computes K and V for its new tokens only and
 * adds them to what is cached; "Features", "Advanced Scheduling" for prompt
 * chunks beside decoding sequences).  Results equal, bit for bit,
 * pa_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping,
 * num_new_rows, ...) followed by pa_mq_attention(...) with the other
 * fields, on `stream`; one launch writes the rows and builds the plan (two
 * launches in the two calls).  num_new_rows may differ from num_tokens
 * (0: no rows).  Errors: those of the two calls, checked before anything is
 * enqueued (where the attention arguments are wrong, the fused step writes
 * no rows, which the two calls would have written first).  Environment
 * PA_STEP_FUSE=0 makes it issue the two calls instead.
 */
typedef struct {
  /* pa_reshape_and_cache (skipped when num_new_rows == 0) */
  const void* key;
  const void* value;
  const int64_t* slot_mapping;
  int num_new_rows;
  /* pa_mq_attention */
  void* out;
  void* workspace;
  size_t workspace_bytes;
  const void* q;
  const int32_t* query_start;
  int num_tokens;
  int max_query_len;
  void* k_cache;
  void* v_cache;
  const int32_t* block_tables;
  int max_blocks_per_seq;
  const int32_t* context_lens;
  int max_context_len;
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int head_dim;
  int block_size;
  int num_blocks;
  float scale;
  float softcap;
  int window;
  int partition_size;
  pa_dtype dtype;
} pa_mq_step_args;

int pa_mq_step(const pa_mq_step_args* args, void* stream);

/*
 * One layer-step: pa_reshape_and_cache (when num_tokens > 0), pa_decode and
 * pa_decode_reduce with the arguments below, on one stream.  The step can
 * also be captured once into a HIP graph and replayed: static graph execution
 * removes the per-launch host cost where it dominates (small batches, short
 * contexts) — the pages list pre-compiled execution plans among the engines'
 * techniques (GeeeekExplorer/nano-vllm on awesome-repositories, "Features":
 * graph compilation, static graph execution).  A replay reads and writes the
 * same buffers as the capture; their contents may change between replays,
 * their addresses and the host-side sizes may not.
 */
typedef struct {
  /* reshape_and_cache (skipped when num_tokens == 0) */
  const void* key;
  const void* value;
  const int64_t* slot_mapping;
  int num_tokens;
  /* decode */
  void* out;
  void* workspace;
  size_t workspace_bytes;
  const void* q;
  void* k_cache;
  void* v_cache;
  const int32_t* block_tables;
  int max_blocks_per_seq;
  const int32_t* context_lens;
  int max_context_len;
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int head_dim;
  int block_size;
  int num_blocks;
  float scale;
  float softcap;
  int window;
  int partition_size;
  pa_dtype dtype;
  /* nonzero: a decode step's one new token per sequence -- num_tokens ==
     num_seqs and row i of key/value is the newest token of sequence i
     (position context_lens[i] - 1), with slot_mapping[i] its slot or -1
     (-1 also for a sequence with context_lens[i] == 0, which has none).
     Then the decode launch writes the rows itself (vector kernel) and no
     launch runs before it for them.  Results are the same bits either way;
     rows that break the contract give undefined results. */
  int new_rows_at_tails;
} pa_step_args;

/*
 * Runs the step on `stream` (no graph).  Returns the first failing status;
 * argument errors are those of the three calls.  The results are those of
 * the three calls in turn, bit for bit: one launch writes the new K/V rows
 * and builds the sequence order (two launches in the three calls), then the
 * decode kernel and (keys split) the reduce kernel run.  Environment
 * PA_STEP_FUSE=0 makes it issue the three calls instead.
 */
int pa_step(const pa_step_args* args, void* stream);

typedef struct pa_step_graph pa_step_graph; /* opaque */

/*
 * Captures the step on `stream` (which must not be capturing already) into a
 * graph and instantiates it.  Set-up call: it allocates host-side graph
 * objects, nothing on the device; free them with pa_step_graph_destroy.
 * Nothing is executed during capture.  *graph is set only on success.
 */
int pa_step_graph_create(const pa_step_args* args, void* stream, pa_step_graph** graph);

/*
 * Captures num_steps layer-steps, args[0] .. args[num_steps - 1] in this
 * order, into one graph, e.g. the attention of every layer of a model for
 * one decode step: a replay then runs them all from one launch, so the
 * per-launch cost of a graph is paid once for all of them.  The steps run
 * one after another on the stream, as the same pa_step calls would; each
 * needs its own workspace unless they run strictly in order (they do: a
 * graph replays them in capture order).  Arguments, errors and ownership as
 * pa_step_graph_create (which is this call with num_steps = 1).
 */
int pa_step_graph_create_n(const pa_step_args* args, int num_steps, void* stream,
                           pa_step_graph** graph);

/* Enqueues one replay of the captured step(s) on `stream`. */
int pa_step_graph_launch(pa_step_graph* graph, void* stream);

/* Frees the graph (NULL is a no-op). */
int pa_step_graph_destroy(pa_step_graph* graph);

/* Size of the scratch array pa_step_static uses, per GPU (128 MiB). */
#define PA_STATIC_SCRATCH_BYTES ((size_t)128 << 20)

/*
 * pa_step without a caller workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc.  The step's scratch (sequence order, work list,
 * split-K partials) lives in a file-scope device array of
 * PA_STATIC_SCRATCH_BYTES bytes, one per GPU, held from the first call on
 * that GPU until the process ends; args->workspace and
 * args->workspace_bytes are ignored.  The array's device address is looked
 * up once per device, on the first call with that device current (`stream`
 * must belong to the current device).  Returns PA_ESCRATCH, before anything
 * is enqueued, when pa_decode_workspace_size for the arguments exceeds
 * PA_STATIC_SCRATCH_BYTES; otherwise the status and results of pa_step, bit
 * for bit.  Nothing here allocates or frees.  Every call on one GPU shares
 * that GPU's array and nothing in it needs to start at zero (each step
 * writes what it reads): calls that may overlap on one GPU -- on different
 * streams, or from several host threads -- race, so issue them on one
 * stream.
 */
int pa_step_static(const pa_step_args* args, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
