/*
 * ak.h -- C ABI of the paged-KV attention library (libak.so) for AMD MI355X (gfx950).
 *
 * The library computes one step of batched attention over a paged KV cache:
 *   1. ak_store_kv  scatters this step's new K/V rows into cache slots;
 *   2. ak_plan      compiles the ragged batch (CSR page table + query offsets)
 *                   into a work list and split-KV partition, once per step;
 *   3. ak_run       runs GQA attention for every layer with that plan (decode
 *                   and causal extend/prefill in one call), merging split-KV
 *                   partial states by their log-sum-exp.
 *
 * Sources (page title, section):
 *   - "vLLM attention backend" (pinghaoyang.com.cn): "plan() and run()", "From a
 *     2-D block table to a CSR page table", "Write the KV first", the worked
 *     example with requests A/B/C, "Nine invariants".
 *   - "SGLang attention backend" (pinghaoyang.com.cn): the kv_indptr / kv_indices /
 *     kv_last_page_len triple, "Why metadata is built once per step",
 *     "The two forms of extend" (state merge), "Where masks come from".
 *   - mini-sglang handbook, "GPU attention": "FlashInfer: plan and run" and the CPU
 *     reference paged attention of "Verify on the CPU".
 *   - "FlashInfer and the backend abstraction" (mlinterviewnotes.com): "plan()",
 *     "Fail loudly".
 *
 * Conventions shared by every entry point
 *   - Every call returns ak_status; no exception or abort crosses the ABI.  On
 *     failure ak_last_error() returns a message for the calling thread.
 *   - Device pointers are HIP device memory on the current device.  Host pointers
 *     are ordinary process memory.  The caller owns every buffer it passes; the
 *     library never frees caller memory.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Kernels are
 *     enqueued asynchronously on it; errors detected on the host are returned
 *     before anything is enqueued.
 *   - Anything outside the supported set returns AK_ERR_UNSUPPORTED; the library
 *     never substitutes another method ("Fail loudly").
 */
#ifndef AK_H_
#define AK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  AK_OK = 0,
  AK_ERR_INVALID_ARG = -1,     /* null pointer, negative size, bad enum value    */
  AK_ERR_UNSUPPORTED = -2,     /* valid request outside the supported set        */
  AK_ERR_BAD_INDPTR = -3,      /* an indptr array does not start at 0 or decreases */
  AK_ERR_BAD_LENGTHS = -4,     /* last_page_len out of [1, B], query longer than KV */
  AK_ERR_SHAPE_MISMATCH = -5,  /* tensor shapes disagree with each other or the plan */
  AK_ERR_HIP = -6,             /* a HIP runtime call failed                      */
  AK_ERR_OOM = -7              /* device or host allocation failed               */
} ak_status;

typedef enum {
  AK_F32 = 0,       /* IEEE binary32                                              */
  AK_BF16 = 1,      /* bfloat16                                                   */
  AK_FP8_E4M3 = 2,  /* OCP FP8 E4M3 ("fn": no inf, max 448), value = code * scale */
  AK_I32 = 3,
  AK_I64 = 4
} ak_dtype;

/* A strided view of device memory.  shape/stride use the first `ndim` entries;
 * strides are in elements.  `scale` is read only for AK_FP8_E4M3. */
typedef struct {
  void* data;
  int32_t dtype;     /* ak_dtype */
  int32_t ndim;
  int64_t shape[4];
  int64_t stride[4];
  float scale;
} ak_tensor;

/* ------------------------------------------------------------------ store */

/* ak_store_kv -- write this step's K/V into the paged cache by slot.
 *
 * Defines ("vLLM attention backend", "Write the KV first"; worked example):
 * for every new token i with slot_mapping[i] >= 0, flat cache row
 * slot_mapping[i] (page = slot / B, offset = slot % B) receives k[i] in
 * k_cache and v[i] in v_cache.  The store is a separate call that must be
 * enqueued before the ak_run that reads those rows, so decode, extend and
 * prefill all attend over one cache under a causal bound.
 *
 *   k, v          [N, Hkv, D]  F32 or BF16, D contiguous (stride 1).
 *   slot_mapping  [N]          I64 device array; negative = padding, skipped.
 *   k_cache,
 *   v_cache       [P, B, Hkv, D]  F32, BF16 or FP8_E4M3, D contiguous.
 *
 * Conversions: equal dtypes copy bits; F32 -> BF16 rounds to nearest even;
 * F32/BF16 -> FP8_E4M3 computes the binary32 quotient x / cache.scale, rounds it
 * to nearest even E4M3 and saturates to +-448 (the sign of a zero result is
 * kept).  BF16 -> F32 and writes into a narrower-than-FP8 type are unsupported.
 * Every slot must lie in [0, P*B) or be negative; two tokens with the same slot
 * in one call leave either value (the pages' invariants forbid it).
 * Errors: AK_ERR_INVALID_ARG (null data, ndim), AK_ERR_SHAPE_MISMATCH (N, Hkv, D
 * disagree), AK_ERR_UNSUPPORTED (dtype pair), AK_ERR_HIP (launch failure).
 * N = 0 returns AK_OK and launches nothing. */
ak_status ak_store_kv(const ak_tensor* k, const ak_tensor* v, const ak_tensor* slot_mapping,
                      ak_tensor* k_cache, ak_tensor* v_cache, void* stream);

/* --------------------------------------------------------------- metadata */

/* ak_csr_from_block_table -- the CSR page table of a batch from its 2-D block
 * table, on the device.
 *
 * Defines ("vLLM attention backend", "From a 2-D block table to a CSR page
 * table"; checked against the page's worked example): request r owns the first
 * pages_r = ceil(L_r / B) kernel pages of its block-table row, and
 *   kv_indptr[0] = 0,  kv_indptr[r + 1] = kv_indptr[r] + pages_r,
 *   kv_indices[kv_indptr[r] + k] = block_table[r][k / ratio] * ratio + k % ratio
 *                                  for k < pages_r,
 *   last_page_len[r] = L_r - (pages_r - 1) * B  (in [1, B]; 0 when L_r = 0).
 * block_ratio = 1 copies the row.  block_ratio > 1 is the same page's "Hybrid
 * KV and virtual kernel blocks": the table holds manager blocks of
 * block_ratio * B tokens, and manager block b of a cache [P, ratio * B, Hkv, D]
 * is kernel pages b * ratio .. b * ratio + ratio - 1 of that cache viewed as
 * [P * ratio, B, Hkv, D] (the view ak_run then reads).
 *
 *   block_table    device int32 [batch_size, max_blocks], row-major, rows
 *                  contiguous; entries past the blocks that cover L_r are never
 *                  read.
 *   seq_lens       device int32 [batch_size], the KV length L_r of each request
 *                  (this step's tokens included).  A length outside
 *                  [0, max_blocks * block_ratio * B] is clamped into it (the
 *                  row holds no more).
 *   kv_indptr      device int32 [batch_size + 1], written.
 *   kv_indices     device int32 [capacity], written in [0, kv_indptr[batch_size]);
 *                  entries at or past `capacity` are dropped, so a caller that
 *                  cannot bound the total reads kv_indptr[batch_size] back.
 *   last_page_len  device int32 [batch_size], written.
 *
 * Outputs are caller-owned; the result is the plain definition above, bit for
 * bit (integer work).  Page ids are copied unchecked.  Enqueued on `stream`,
 * no host synchronisation, no allocation.  Errors: AK_ERR_INVALID_ARG (null
 * pointer, batch_size < 0, page_size < 1, block_ratio < 1, max_blocks < 0,
 * capacity < 0), AK_ERR_UNSUPPORTED (block_ratio * page_size > 2^20 or
 * max_blocks * block_ratio > 2^31 - 1), AK_ERR_HIP.  batch_size = 0 writes
 * kv_indptr[0] = 0 only. */
ak_status ak_csr_from_block_table(const int32_t* block_table, int64_t max_blocks,
                                  const int32_t* seq_lens, int32_t batch_size, int32_t page_size,
                                  int32_t block_ratio,
                                  int32_t* kv_indptr, int32_t* kv_indices, int64_t capacity,
                                  int32_t* last_page_len, void* stream);

/* ak_slot_mapping -- the cache slot of every new token of a step, on the device.
 *
 * Defines ("vLLM attention backend", "Write the KV first" and the worked
 * example: position 127 of a request whose eighth page is 10 lands in slot 175
 * for B = 16): the n_r = qo_indptr[r + 1] - qo_indptr[r] new tokens of request
 * r are its last n_r positions, so token qo_indptr[r] + j has position
 * p = L_r - n_r + j and slot block_table[r][p / B] * B + p % B.
 *
 *   block_table   device int32 [batch_size, max_pages], as above (with manager
 *                 blocks, pass their size as page_size: the slot is the same).
 *   qo_indptr     device int32 [batch_size + 1], starting at 0, non-decreasing.
 *   seq_lens      device int32 [batch_size], L_r with this step's tokens.
 *   slot_mapping  device int64 [num_tokens], written: the slot, or -1 for a
 *                 token past qo_indptr[batch_size] (padding of a fixed-size
 *                 batch) and for a position outside [0, max_pages * B).  The
 *                 result feeds ak_store_kv, which skips negative slots.
 *
 * Enqueued on `stream`; no synchronisation, no allocation.  Errors:
 * AK_ERR_INVALID_ARG (null pointer, negative size, page_size < 1), AK_ERR_HIP.
 * num_tokens = 0 launches nothing. */
ak_status ak_slot_mapping(const int32_t* block_table, int64_t max_pages, const int32_t* qo_indptr,
                          const int32_t* seq_lens, int32_t batch_size, int32_t page_size,
                          int64_t* slot_mapping, int64_t num_tokens, void* stream);

/* ------------------------------------------------------------------- plan */

typedef struct ak_plan_t ak_plan_t;    /* opaque; owned by the library */

enum {
  AK_PLAN_HOST_ONLY = 1,        /* build the work list without touching the GPU           */
  AK_PLAN_MERGE_IN_KERNEL = 2,  /* split decode units (<= 16 rows) are merged by the last of
                                   their parts inside the attention kernel (bf16 q) instead
                                   of by a separate merge launch: one launch fewer per run,
                                   for launch-bound small batches; slower for large ones  */
  AK_PLAN_SHARED_PAGES = 4,     /* requests of the batch share pages (a common prefix): decode
                                   reads K/V with ordinary cached loads so later readers of a
                                   shared page hit the caches; by default they are streamed
                                   (read once, kept out of the caches)                    */
  AK_PLAN_STREAM_K = 8          /* stream-K decode ("SGLang attention backend", the lean-decode
                                   metadata of "Other backends' metadata"): the decode units'
                                   KV ranges, laid end to end, are cut into equal contiguous
                                   shares, one per resident workgroup (two per compute
                                   unit); each workgroup of one persistent launch works
                                   through the pieces of its share, and a unit cut across
                                   shares is merged from their partial states.  Not for
                                   fixed plans                                             */
};

typedef struct {
  float sm_scale;        /* softmax scale; <= 0 selects 1/sqrt(head_dim)            */
  int32_t num_cus;       /* compute units to balance for; 0 = ask the device (256
                            in host-only plans)                                    */
  int32_t max_splits;    /* bound on KV splits per (request, KV head); 0 = 64.  Exceeded
                            only when a split would span more than 1024 pages (page
                            size 1 or 2 with long contexts)                        */
  int32_t min_chunk;     /* smallest KV split in tokens; 0 = library default       */
  int32_t flags;         /* AK_PLAN_HOST_ONLY | AK_PLAN_MERGE_IN_KERNEL |
                            AK_PLAN_SHARED_PAGES | AK_PLAN_STREAM_K                  */
  void* stream;          /* stream for the plan's upload; NULL = default stream     */
} ak_plan_opts;

/* ak_plan -- compile one batch's metadata into a reusable plan.
 *
 * Defines ("vLLM attention backend", "plan() and run()" and "From a 2-D block
 * table to a CSR page table"; "SGLang attention backend", the kv_indptr /
 * kv_indices / kv_last_page_len triple; mini-sglang "FlashInfer: plan and run"):
 * request r owns query rows qo_indptr[r] .. qo_indptr[r+1]-1 of q and the pages
 * kv_indices[kv_indptr[r] .. kv_indptr[r+1]-1]; its KV length is
 *   L_r = (kv_indptr[r+1] - kv_indptr[r] - 1) * page_size + last_page_len[r]
 * (0 when it has no pages), and its n_r queries sit at positions L_r - n_r + j.
 * Query head h reads KV head h / (num_qo_heads / num_kv_heads).
 *
 *   qo_indptr      host int32 [batch_size + 1]   (copied)
 *   kv_indptr      host int32 [batch_size + 1]   (copied)
 *   kv_indices     DEVICE int32 [kv_indptr[batch_size]]  physical page ids;
 *                  borrowed, not read by ak_plan: it must stay allocated and
 *                  unchanged until the last ak_run with this plan.
 *   last_page_len  host int32 [batch_size]        (copied); in [1, page_size]
 *                  for a request with pages, ignored for one without.
 *   causal         1: key t is visible to a query at position p iff t <= p;
 *                  0: all keys are visible (then n_r may exceed L_r, and a
 *                  request without pages yields the empty state: out 0,
 *                  lse -inf -- the prefix segment of a two-segment extend).
 *   window         -1: none; w >= 0 (causal only): keys t >= p - w stay visible,
 *                  i.e. w + 1 keys including the query's own position.
 *   opts           may be NULL.
 *   plan           receives the new plan.
 *
 * The plan reads only host arrays (no device read-back) and makes one
 * host-to-device copy of its work list.  Its device workspace and pinned
 * staging come from a small per-process pool of recycled workspaces; when the
 * host has more than 16 plans' work still queued on the device, ak_plan waits
 * for the oldest of it to finish before reusing its workspace.  Supported: num_qo_heads a multiple of
 * num_kv_heads with a group of 1, 2, 4, 8 or 16; head_dim 64 or 128; page_size
 * a power of two in [1, 256].  Errors: AK_ERR_INVALID_ARG, AK_ERR_UNSUPPORTED,
 * AK_ERR_BAD_INDPTR (qo/kv indptr not starting at 0 or decreasing),
 * AK_ERR_BAD_LENGTHS (last_page_len outside [1, page_size]; with causal = 1,
 * n_r > L_r, including queries on a request without pages), AK_ERR_OOM, AK_ERR_HIP.  batch_size = 0 or no
 * query rows gives a valid empty plan. */
ak_status ak_plan(const int32_t* qo_indptr, const int32_t* kv_indptr, const int32_t* kv_indices,
                  const int32_t* last_page_len, int32_t batch_size, int32_t num_qo_heads,
                  int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t causal,
                  int32_t window, const ak_plan_opts* opts, ak_plan_t** plan);

/* ak_plan_destroy -- release a plan's host memory and device workspace.
 * Waits for nothing: the caller must ensure no ak_run using it is still
 * executing (synchronise the stream first).  NULL is accepted. */
void ak_plan_destroy(ak_plan_t* plan);

/* -------------------------------------------------------------------- run */

/* ak_run -- attention for one layer with a plan.
 *
 * Defines (mini-sglang "Verify on the CPU" reference paged attention; "SGLang
 * attention backend", "Where masks come from" and "The two forms of extend"):
 * for query row i of request r at position p and query head h,
 *   s_t   = sm_scale * q[i,h,:] . K_r[t, h/G, :]   for visible keys t,
 *   out   = sum_t exp(s_t - m) V_r[t, h/G, :] / sum_t exp(s_t - m),
 *   lse   = m + ln sum_t exp(s_t - m)              (natural log),
 * with K_r[t] read from row kv_indices[kv_indptr[r] + t / B] * B + t % B of the
 * cache.  A (request, KV head) whose keys the plan split into S > 1 parts is
 * finished by merging the parts' (out, lse) states: m = max lse_s,
 * out = sum_s e^(lse_s - m) out_s / sum_s e^(lse_s - m).
 *
 *   q        [T, Hq, D]   F32 or BF16, T = qo_indptr[batch_size], D contiguous.
 *   k_cache,
 *   v_cache  [P, B, Hkv, D] same dtype as q, or FP8_E4M3 with BF16 q (the
 *            tensors' scale fields are the per-tensor dequantisation scales);
 *            strides non-negative, rows 16-byte aligned, page and head strides
 *            below 2 GiB and the slot stride times 256 below 2 GiB (in bytes).
 *   out      [T, Hq, D]   dtype of q (never FP8), D contiguous; written.
 *   lse      [T, Hq]      F32, or NULL; written.
 *
 * Every row of out/lse that belongs to a request with n_r > 0 is written.
 * A plan may be run any number of times (once per layer) on one stream; runs
 * sharing a plan must not overlap in time (they share its split workspace).
 * Errors: AK_ERR_INVALID_ARG (null plan/tensor, host-only plan),
 * AK_ERR_SHAPE_MISMATCH (T, Hq, Hkv, D or B disagree with the plan -- a plan
 * built for fewer heads is rejected, never run), AK_ERR_UNSUPPORTED (dtype
 * combination, misaligned rows, cache strides out of range), AK_ERR_HIP.  An empty plan returns AK_OK and
 * launches nothing.  With a fixed plan (ak_plan_fixed) T is the plan's
 * max_tokens, the launches cover its whole capacity whatever the live batch,
 * and rows past qo_indptr[batch_size] of the last update are left untouched. */
ak_status ak_run(const ak_plan_t* plan, const ak_tensor* q, const ak_tensor* k_cache,
                 const ak_tensor* v_cache, ak_tensor* out, ak_tensor* lse, void* stream);

/* ak_run_noalloc -- plan and run one layer in a single call that allocates
 * nothing, for callers that cannot allocate: code under stream capture, tight
 * serving loops, harnesses that forbid hipMalloc.
 *
 * Computes exactly what ak_plan followed by ak_run computes with the same
 * arguments (same work list, same kernels, bitwise the same out and lse); the
 * arguments mean what they mean there, `opts->stream` is ignored and `stream`
 * carries both the metadata upload and the kernels.  Instead of a plan
 * workspace, the work list, merge list, arrival counters and split partials
 * live in one fixed device array of 64 MiB that the library holds on every
 * device it runs on until the process ends; a batch whose work list and split
 * partials need more returns AK_ERR_UNSUPPORTED before anything is enqueued
 * (use ak_plan + ak_run for it).  No device or pinned memory is allocated and
 * nothing is freed; the work list is copied from pageable host memory, which
 * may wait for earlier work on `stream`.  Every call on one device shares that
 * array: calls that overlap in time on one device (different streams, or
 * several host threads) race and must be serialised by the caller; calls on one
 * stream are ordered.  Errors: those of ak_plan and ak_run, and AK_ERR_HIP if
 * the array's device address cannot be obtained. */
ak_status ak_run_noalloc(const int32_t* qo_indptr, const int32_t* kv_indptr,
                         const int32_t* kv_indices, const int32_t* last_page_len,
                         int32_t batch_size, int32_t num_qo_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t page_size, int32_t causal, int32_t window,
                         const ak_plan_opts* opts, const ak_tensor* q, const ak_tensor* k_cache,
                         const ak_tensor* v_cache, ak_tensor* out, ak_tensor* lse, void* stream);

/* ----------------------------------------------------------- diagnostics */

/* Thread-local text of the last error (empty string if none).  Owned by the
 * library; valid until the next ak_* call on the same thread. */
const char* ak_last_error(void);

/* ak_merge_states -- combine two attention states computed over disjoint key
 * sets of the same queries ("SGLang attention backend", "The two forms of
 * extend": the prefix/new-token split of an extend step; the shared-prefix
 * cascade of "vLLM attention backend").  For every (token i, head h):
 *   m   = max(lse_a, lse_b),  w_x = exp(lse_x - m),
 *   out = (w_a * o_a + w_b * o_b) / (w_a + w_b),   lse = m + ln(w_a + w_b),
 * where a state with lse = -inf (no visible key) weighs 0; if both are -inf the
 * output row is 0 and lse is -inf.
 *
 *   o_a, o_b   [T, H, D]  F32 or BF16 (both the dtype of out), D contiguous,
 *              rows 16-byte aligned; each is normalised (an ak_run output).
 *   lse_a,
 *   lse_b      [T, H]     F32, natural log (as ak_run writes it).
 *   out        [T, H, D]  F32 or BF16; may be the same tensor as o_a or o_b
 *              (each row is read before it is written).
 *   lse_out    [T, H]     F32 or NULL; may alias lse_a or lse_b.
 *
 * D must be 64 or 128.  Arithmetic in fp32.  Errors: AK_ERR_INVALID_ARG (null
 * tensor or data), AK_ERR_SHAPE_MISMATCH (shapes disagree), AK_ERR_UNSUPPORTED
 * (dtype, D, layout), AK_ERR_HIP.  T = 0 or H = 0 launches nothing. */
ak_status ak_merge_states(const ak_tensor* o_a, const ak_tensor* lse_a, const ak_tensor* o_b,
                          const ak_tensor* lse_b, ak_tensor* out, ak_tensor* lse_out,
                          void* stream);

/* ----------------------------------------------------------- fixed plans */

/* ak_plan_fixed / ak_plan_update -- a plan whose device workspace never moves,
 * for runs captured into a HIP graph.
 *
 * Follows "vLLM attention backend", the graph-capture section (stable device
 * addresses; dynamic content written into stable buffers), "SGLang attention
 * backend", the backend's graph duties (buffers sized by the largest batch,
 * refreshed before each replay; host work kept out of the graph), and the
 * graph section of "FlashInfer and the backend abstraction" (the tail of
 * persistent scheduling metadata cleared so that stale entries write nothing).
 *
 * ak_plan_fixed allocates, once, a workspace sized for any batch of at most
 * max_batch requests, max_tokens query tokens, max_query_len query tokens in any
 * one request (0 = max_tokens; 1 for pure decode, where max_query_len *
 * num_qo_heads / num_kv_heads <= 16 also drops the large-tile launch) and
 * max_pages pages: the work list
 * with room for every split the planner may choose, the split partials and the
 * merge list, all zeroed (a zero entry is padding: its workgroup exits at once).
 * Geometry (heads, head_dim, page_size, causal, window) and opts are fixed with
 * it and follow ak_plan.  `kv_indices` is the DEVICE int32 buffer of max_pages
 * entries that every later batch's page ids are written into (borrowed; stable
 * for the plan's lifetime).  The call synchronises opts->stream; it is never
 * captured.
 *
 * ak_plan_update plans one batch (host arrays as in ak_plan, validated the same
 * way) and writes its work list over the previous one with asynchronous copies
 * on `stream`, padding out entries the previous batch used past the new one's
 * end.  It must be issued on the stream that replays the runs, between replays,
 * and outside capture.  The plan's workspace holds one batch: an update takes
 * effect for every later replay.  Either call on a stream that is being
 * captured returns AK_ERR_INVALID_ARG.
 *
 * ak_run with a fixed plan launches every kernel over the capacity (fixed
 * grids), so a run captured once replays correctly after any update.  Padding
 * workgroups cost a few microseconds per run.
 *
 * The capacity always suffices for page_size >= 8, KV lengths up to
 * max_splits * (1022 * page_size - 128) and num_kv_heads * sum L_r up to
 * 6 * num_cus * 4096; beyond that ak_plan_update may return AK_ERR_UNSUPPORTED
 * and leaves the plan as it was.
 * Errors: AK_ERR_INVALID_ARG (null pointer, negative capacity, update of a
 * non-fixed plan), AK_ERR_UNSUPPORTED, AK_ERR_SHAPE_MISMATCH (batch larger than
 * the capacities), AK_ERR_BAD_INDPTR / AK_ERR_BAD_LENGTHS (as ak_plan),
 * AK_ERR_OOM, AK_ERR_HIP.  With AK_PLAN_HOST_ONLY in opts->flags nothing is
 * allocated or uploaded (for checking the work list and capacities). */
ak_status ak_plan_fixed(int32_t max_batch, int64_t max_tokens, int64_t max_query_len,
                        int64_t max_pages, const int32_t* kv_indices, int32_t num_qo_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t page_size, int32_t causal, int32_t window,
                        const ak_plan_opts* opts, ak_plan_t** plan);
ak_status ak_plan_update(ak_plan_t* plan, const int32_t* qo_indptr, const int32_t* kv_indptr,
                         const int32_t* last_page_len, int32_t batch_size, void* stream);

/* ak_plan_info -- host-side summary of a plan (any plan, host-only included).
 * Writes up to 13 int64 values into `info` (caller-owned host array):
 *   [0] batch_size  [1] total query rows T  [2] work items  [3] small-tile items
 *   [4] large-tile items  [5] split (request, KV head) units  [6] merge jobs
 *   [7] partial rows in the split workspace; for a fixed plan the capacities
 *   [8] small-tile items [9] large-tile items [10] merge jobs [11] partial rows
 *   (0 for other plans); [12] stream-K workgroups (0 for other plans).
 * Errors: AK_ERR_INVALID_ARG. */
ak_status ak_plan_info(const ak_plan_t* plan, int64_t* info, int32_t n);

/* ak_plan_workgroups -- a stream-K plan's workgroup table, for checking: host
 * int32 wg_first[P + 1] such that workgroup g of the decode launch runs the small
 * items wg_first[g] .. wg_first[g+1]-1 (in ak_plan_export's order, small items
 * first).  *count receives P + 1 (0 for plans without AK_PLAN_STREAM_K); a
 * `capacity` below it returns AK_ERR_INVALID_ARG.  Errors: AK_ERR_INVALID_ARG. */
ak_status ak_plan_workgroups(const ak_plan_t* plan, int32_t* wg_first, int64_t capacity,
                             int64_t* count);

/* ak_plan_export -- copy the plan's work list to host memory for checking.
 * Each item is 8 int32: request, kv_head, first row, row count, kv_begin,
 * kv_end, partial base (-1 = writes the output directly), kind (0 small tile,
 * 1 large tile).  Row rho of (request r, KV head hk) is query token
 * qo_indptr[r] + rho / G and query head hk*G + rho % G.  Items are in launch
 * order (small items first); the large items of an ordinary plan with few
 * units are grouped by die and may include empty items (row count 0, kind 1,
 * partial base -1) that hold a dispatch slot and do nothing.  Also writes the
 * per-request KV lengths L_r into `kv_lens` (host int32 [batch_size], may be
 * NULL).  `items` holds `capacity` items; more than that returns
 * AK_ERR_INVALID_ARG with the needed count in *count. */
ak_status ak_plan_export(const ak_plan_t* plan, int32_t* items, int64_t capacity, int64_t* count,
                         int32_t* kv_lens);

/* ak_gather_slots -- the plan's KV indexing, materialised (debug).
 * For every request r and position t < L_r writes the flat cache slot
 * kv_indices[kv_indptr[r] + t / B] * B + t % B ("vLLM attention backend", the
 * worked example's slot formula) into slots[kv_offset_r + t], where kv_offset_r =
 * sum of L over earlier requests.  The slot is computed by the device functions
 * the attention kernels address their K/V rows with -- the page-id read and
 * clamp, then the row offset -- run with a page stride of B and a slot stride of
 * 1 instead of the cache's byte strides: `addressing` 0 selects the decode and
 * fp32 kernels' form (page id clamped as staged, 64-bit row offset), 1 the
 * prefill kernels' load-to-LDS copy form (raw page id clamped at the copy,
 * in-page offset in 32 bits), 2 the same copy form computed entirely in 32 bits
 * with 24-bit multiplies, which the prefill kernels use for pools of at most 2^24
 * pages whose bytes (from a head's base) span at most 4 GiB (page ids are clamped
 * into 2^24 pages here).  `slots` is a device int64 array of at least sum_r L_r
 * entries; the call synchronises the stream.  Errors: AK_ERR_INVALID_ARG (null
 * argument, host-only plan, addressing not 0, 1 or 2), AK_ERR_HIP. */
ak_status ak_gather_slots(const ak_plan_t* plan, int32_t addressing, int64_t* slots, void* stream);

/* ak_fp8_to_bf16 -- the cache's FP8 E4M3 decode, materialised (diagnostics).
 * Widens n E4M3 codes (device uint8 array, n a multiple of 8) into bf16 bit
 * patterns (device uint16 array of n entries) with the conversion the attention
 * kernels apply to FP8 K/V rows before their MFMA (exact, scale 1).
 * Errors: AK_ERR_INVALID_ARG (null pointer, n < 0 or not a multiple of 8),
 * AK_ERR_HIP. */
ak_status ak_fp8_to_bf16(const uint8_t* codes, uint16_t* out, int64_t n, void* stream);

/* Per-kernel timing with HIP events on the launch stream (diagnostics).
 * Kernel kinds: 0 store, 1 small-tile attention, 2 large-tile attention,
 * 3 merge, 4 fp32 attention.  ak_profile_enable(kinds) records an event pair
 * around every launch of the kinds whose bit (1 << kind) is set in `kinds`
 * (0 = off; AK_PROFILE_ALL = every kind; launches during stream capture are
 * never timed).  Each pair adds a few microseconds between kernels, so time
 * only the kinds needed.  ak_profile_read copies, per kind, the launch count and
 * the summed milliseconds measured so far into host arrays of length n, then
 * resets the counters.  Reading synchronises on the events.
 * Errors: AK_ERR_INVALID_ARG (negative mask). */
enum { AK_PROFILE_ALL = 0x1F };
ak_status ak_profile_enable(int32_t kinds);
ak_status ak_profile_read(int64_t* launches, double* total_ms, int32_t n);

/* Library version string. */
const char* ak_version(void);

#ifdef __cplusplus
}
#endif
#endif /* AK_H_ */
