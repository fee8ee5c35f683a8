/*
 * ragged_prefill.h — C ABI of the MI355X (gfx950) ragged prefill attention library.
 *
 * The operation (page "Module flashinfer", module doc and functions
 * ragged_prefill_bf16_hd128 / ragged_prefill_bf16_hd256): N requests of
 * different lengths, located in packed buffers by q_indptr / kv_indptr ragged
 * offsets, run their attention in ONE launch,
 *
 *     O = softmax(sm_scale * Q K^T + mask) V
 *
 * in BF16 with grouped-query heads (num_qo_heads a multiple of num_kv_heads,
 * qo head h reads kv head h / (num_qo_heads / num_kv_heads)), head_dim 128 or
 * 256, causal selectable.  The causal mask is aligned to the end of each
 * request's KV (bottom-right; page "flashinfer-ai/flashinfer", benchmarks
 * README, attention flag --causal): key j is visible to query row i of a
 * request iff j <= i + kv_len - qo_len.  The library also returns the per-row
 * log-sum-exp (the *_return_lse prefill entry points, page
 * "flashinfer-ai/flashinfer", attention API, single request prefill).
 *
 * Layouts (packed NHD, contiguous, device memory, 16-byte aligned base):
 *   q, o : bf16 [total_q,  num_qo_heads, head_dim]
 *   k, v : bf16 [total_kv, num_kv_heads, head_dim]
 *   lse  : fp32 [total_q,  num_qo_heads], natural log of sum_j exp(s_j) over
 *          the visible keys, s_j = sm_scale * q.k_j.  May be NULL.
 *   q_indptr, kv_indptr : HOST int32 [batch + 1], non-decreasing, >= 0;
 *          request b owns q rows [q_indptr[b], q_indptr[b+1]) and kv rows
 *          [kv_indptr[b], kv_indptr[b+1]); q_indptr[0] need not be 0.
 *
 * Conventions:
 *   - Rows outside every request are never written.  A request with
 *     qo_len = 0 writes nothing.
 *   - A query row that sees no key (kv_len = 0, or causal with
 *     i < qo_len - kv_len) gets O = +0 and LSE = -inf.
 *   - batch == 0 or total_q == 0 returns RP_OK without launching anything
 *     (the empty-batch early return of page "vllm-rlt PR #112", design notes).
 *   - Output rounding: fp32 -> bf16 round-to-nearest-even, once.
 *   - Per-request results are bit-for-bit independent of the other requests
 *     in the batch and of how the planner places the work.
 *   - All device work is enqueued on `stream` (a hipStream_t; NULL = the
 *     null stream).  Asynchronous device faults surface at the caller's next
 *     synchronisation.
 *   - Nothing throws across this boundary; every entry point returns a
 *     status.  rp_last_error() gives a thread-local description of the last
 *     failure.
 *
 * Ownership: the caller owns q, k, v, o, lse, the indptr arrays and the
 * stream; the library never frees them.  A plan owns its host metadata and its
 * device-resident worklist; destroy it only after the stream work that uses it
 * has completed.  The workspace of the two-phase API is caller-provided (the
 * "instance-owned workspace" of page "vllm-rlt PR #112", design notes and
 * review); the one-shot call keeps workspaces of its own, one per (device,
 * stream), grown on first use and kept until the process ends.
 */
#ifndef RAGGED_PREFILL_H
#define RAGGED_PREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RP_ABI_VERSION 7

/* Status codes. */
enum rp_status {
    RP_OK = 0,
    RP_EINVAL = -1,        /* malformed argument (pointer, shape, offsets, scale) */
    RP_EUNSUPPORTED = -2,  /* valid but not supported (head_dim, device) */
    RP_ENOMEM = -3,        /* host or device allocation failed; outputs untouched */
    RP_EDEVICE = -4        /* a HIP runtime call or a launch failed */
};

/* Static text for a status code; never NULL. */
const char *rp_status_string(int status);

/* Thread-local text describing the last failure on this thread ("" if none). */
const char *rp_last_error(void);

/* RP_ABI_VERSION of the loaded library. */
int rp_abi_version(void);

/* 1 if the current HIP device is a gfx950 and the kernels are loadable, else 0
 * (the available() gate of page "Module flashinfer", functions). */
int rp_available(void);

/*
 * One-shot call: plans and runs on `stream` (the ragged_prefill_bf16_hd128 /
 * _hd256 FFI of page "Module flashinfer", with head_dim an argument).
 * head_dim must be 128 or 256; num_qo_heads % num_kv_heads == 0;
 * sm_scale finite.  Plans are cached per (device, offsets, shape), at most 8
 * per device; the split-KV workspace is library-owned, one per (device,
 * stream), at most 8 streams per device.
 *
 * Streams: calls enqueued on different streams use different workspaces, so
 * they may run concurrently; calls on one stream are ordered by it.  The
 * upload of a new plan's worklist is synchronous; growing a stream's
 * workspace waits for that stream; evicting a cached plan or a stream's
 * workspace waits for the device.  Calls from several host threads are
 * serialised by the library.
 *
 * HIP graph capture: a call on a capturing stream must find its plan cached
 * and its stream's workspace large enough (an earlier call with the same
 * offsets on that stream ensures both); otherwise it returns RP_EINVAL and
 * enqueues nothing.  A captured graph keeps using that plan and workspace:
 * later one-shot calls that would evict them (more than 8 distinct plans or
 * streams on the device) must not run while the graph may still be
 * replayed.  The two-phase API has none of these limits.
 */
int ragged_prefill_bf16(const void *q, const void *k, const void *v, void *o, float *lse,
                        const int32_t *q_indptr, const int32_t *kv_indptr, int batch,
                        int num_qo_heads, int num_kv_heads, int head_dim, int causal,
                        float sm_scale, void *stream);

/* ---- Two-phase API: plan once per batch shape, run many times ---------------
 * ("preparation once per KV batch", page "vllm-rlt PR #112", review item 3.)
 */

typedef struct rp_plan rp_plan;

/* Placement of tiles whose visible keys span more than one canonical KV
 * chunk.  Either way each chunk's state is computed from a fresh start and
 * the states are folded in ascending chunk order with the same arithmetic
 * (merge of attention states, page "flashinfer-ai/flashinfer", "Merge
 * Attention States"; split-KV scheduled automatically, same page, attention
 * API, task-scheduled attention), so the three modes give identical bits. */
enum rp_split_mode {
    RP_SPLIT_AUTO = 0,    /* NEVER at head_dim 128 when the longest folded tile costs no more
                             than the average load of the 512 workgroups resident on the GPU
                             (the grid fills it without split-KV); ALWAYS otherwise */
    RP_SPLIT_NEVER = 1,   /* one workgroup per tile runs its chunks in order and folds their
                             states itself (running state in a workspace slot, no merge kernel) */
    RP_SPLIT_ALWAYS = 2   /* one workgroup per (tile, KV chunk) + merge kernel */
};

/* Planner options.  All-zero means defaults.  The KV chunk size fixes the
 * numerics (where partial states are cut and merged); the split mode only
 * moves work between workgroups and never changes a bit of the results. */
typedef struct rp_plan_opts {
    int kv_chunk;    /* canonical KV chunk in keys (multiple of 64, >= 64); 0 = default 8192 */
    int split_mode;  /* enum rp_split_mode */
    int host_only;   /* nonzero: plan on the host only; such a plan can be inspected, not run */
    int num_xcds;    /* XCDs the launch order is arranged for (workgroup b runs on XCD
                        b % num_xcds); 0 = default (8, the MI355X XCD count),
                        1 = plain longest-first order */
} rp_plan_opts;

/* Summary of a plan (host side). */
typedef struct rp_plan_info {
    int64_t num_items;         /* tile work items (workgroups of the tile kernel) */
    int64_t num_partial_items; /* of which write fp32 partial states */
    int64_t num_merge_items;   /* merge kernel workgroups (tiles with partial states) */
    int64_t total_q;           /* sum of qo_len */
    int64_t total_kv;          /* sum of kv_len */
    int32_t tile_rows;         /* rows (token x qo-head pairs) per tile */
    int32_t tile_tokens;       /* tokens per tile */
    int32_t key_block;         /* keys per inner-loop block */
    int32_t kv_chunk;          /* canonical KV chunk, keys */
    double flops;              /* algorithmic: 4 * head_dim * num_qo_heads * visible pairs */
    double bytes;              /* algorithmic: Q,K,V read once, O,LSE written once */
    size_t workspace_bytes;    /* bytes rp_run needs (0 if no partial states) */
    int64_t num_fold_items;    /* of num_items, those that fold their tile's KV chunks */
} rp_plan_info;

/* Build a plan from HOST offsets.  On success *out owns a plan (possibly with
 * zero items for an empty batch).  Unless opts->host_only, the worklist is
 * copied to the current device (synchronously). */
int rp_plan_create(const int32_t *q_indptr, const int32_t *kv_indptr, int batch,
                   int num_qo_heads, int num_kv_heads, int head_dim, int causal,
                   const rp_plan_opts *opts, rp_plan **out);

int rp_plan_get_info(const rp_plan *plan, rp_plan_info *info);

/* Device workspace bytes rp_run needs for this plan (0 = none). */
size_t rp_plan_workspace_bytes(const rp_plan *plan);

/* Host copy of the tile worklist: RP_ITEM_INTS int32 per item, in launch
 * order (for inspection and tests); items with n_tok = 0 (second int) are
 * padding that does nothing.  capacity counts items.  Returns the number of
 * items copied (>= 0) or a negative status. */
#define RP_ITEM_INTS 16
int64_t rp_plan_copy_items(const rp_plan *plan, int32_t *dst, int64_t capacity);

/* Run a plan on `stream`.  workspace: device memory of at least
 * rp_plan_workspace_bytes(plan) bytes, 256-byte aligned (may be NULL when that
 * is 0).  Launches one tile kernel, plus one merge kernel when the plan holds
 * partial states.  Captures into a HIP graph (no allocation, no host sync, no
 * memset). */
int rp_run(const rp_plan *plan, const void *q, const void *k, const void *v, void *o,
           float *lse, float sm_scale, void *workspace, size_t workspace_bytes,
           void *stream);

/* rp_run for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * kernels, with the split-KV partial states in a fixed array of the library
 * (a 32 MiB __device__ object that every device the library runs on holds
 * until the process ends) instead of a caller workspace.  The plan must come
 * from rp_plan_create (run on this device) and need at most 32 MiB of
 * workspace (rp_plan_workspace_bytes), else RP_EUNSUPPORTED and nothing is
 * enqueued; plans without split KV need none.  No allocation, free or host
 * synchronisation happens in the call.  Calls on one device share the array:
 * calls that overlap in time (other streams, other host threads) race on it.
 * Everything else as for rp_run. */
int rp_run_noalloc(const rp_plan *plan, const void *q, const void *k, const void *v, void *o,
                   float *lse, float sm_scale, void *stream);

/* Run a plan over PAGED K/V (append prefill over a KV cache; paged KV cache
 * prefill of page "flashinfer-ai/flashinfer", attention API, and the block
 * tables, page sizes and NHD layout of page "vllm-rlt PR #112", design
 * notes).  The plan is the same as for rp_run (built from the kv lengths in
 * kv_indptr; the offsets themselves are not used here).
 *   k_pages, v_pages: bf16 page pools [num_pages][page_size][num_kv_heads]
 *     [head_dim], contiguous, 16-byte aligned, device.
 *   block_table: int32 [batch][max_blocks_per_seq], device: key j of request
 *     b is slot j % page_size of page block_table[b][j / page_size].  Entries
 *     are clamped to >= 0 when read, and entries past a request's
 *     ceil(kv_len / page_size) pages are never read, so padding (-1, 0, stale
 *     ids) is invisible.  Every entry that is read must name a page inside
 *     the pools (not checked).
 *   page_size: 16, 32, 64 or 128 keys.  max_blocks_per_seq must be at least
 *     ceil(max kv_len / page_size), else RP_EINVAL.
 * Everything else (q, o, lse, sm_scale, workspace, stream, ordering) is as for
 * rp_run; results are bit-identical to rp_run on the same keys stored
 * contiguously. */
int rp_run_paged(const rp_plan *plan, const void *q, const void *k_pages, const void *v_pages,
                 const int32_t *block_table, int max_blocks_per_seq, int page_size, void *o,
                 float *lse, float sm_scale, void *workspace, size_t workspace_bytes,
                 void *stream);

/* FP8 K/V (the FP8 KV cache of page "flashinfer-ai/flashinfer", benchmarks
 * README, attention flags --q_dtype / --kv_dtype fp8_e4m3): k and v hold OCP
 * FP8 E4M3 codes (one byte per element, same NHD layout and offsets as
 * rp_run, 16-byte aligned), dequantised as code x k_scale and code x
 * v_scale (per-tensor scales, finite).  Q, O and LSE are as for rp_run (bf16
 * Q and O).  The result is the attention over the dequantised K and V; the
 * E4M3 codes convert to bf16 exactly, k_scale is folded into the softmax
 * scale and v_scale into the output normalisation.  Both head dims of the
 * plan (128, 256) are supported.  Codes 0x7f / 0xff (NaN) give NaN. */
int rp_run_fp8kv(const rp_plan *plan, const void *q, const void *k_fp8, const void *v_fp8,
                 float k_scale, float v_scale, void *o, float *lse, float sm_scale,
                 void *workspace, size_t workspace_bytes, void *stream);

/* rp_run_paged with FP8 (E4M3) page pools [num_pages][page_size]
 * [num_kv_heads][head_dim] bytes; scales and limits as for rp_run_fp8kv. */
int rp_run_paged_fp8kv(const rp_plan *plan, const void *q, const void *k_pages, const void *v_pages,
                       const int32_t *block_table, int max_blocks_per_seq, int page_size,
                       float k_scale, float v_scale, void *o, float *lse, float sm_scale,
                       void *workspace, size_t workspace_bytes, void *stream);

/* Destroys a plan of either kind (a shared-prefix plan frees both levels). */
void rp_plan_destroy(rp_plan *plan);

/* ---- Attention states and shared-prefix (cascade) attention ----------------
 * An attention state of a query row and qo head over a key set is (v, s): v
 * the softmax-weighted mean of the values over that set (bf16 [head_dim]),
 * s the natural-log log-sum-exp of its scores (fp32), i.e. exactly the O and
 * LSE that rp_run returns.  States over disjoint key sets merge into the state
 * over their union (page "flashinfer-ai/flashinfer", cascade API, Merge
 * Attention States):
 *     s = log(sum_i exp(s_i)),   v = sum_i exp(s_i - s) v_i,
 * computed in fp32 in ascending state order, v rounded to bf16 (RNE) once.
 * A state with s = -inf (empty key set) contributes nothing; if every state
 * is empty the result is v = +0, s = -inf.
 * Layouts are contiguous, device memory, v pointers 16-byte aligned:
 *   v: bf16 [rows][num_heads][head_dim], s: fp32 [rows][num_heads];
 *   head_dim a power of two in [8, 512]; num_heads in [1, 65535].
 * s_out may be NULL (LSE not wanted).  Inputs and outputs may alias exactly
 * (same pointer) but must not otherwise overlap.  Enqueued on `stream`;
 * rows == 0 returns RP_OK without launching. */
int rp_merge_state(const void *v_a, const float *s_a, const void *v_b, const float *s_b,
                   void *v_out, float *s_out, int64_t rows, int num_heads, int head_dim,
                   void *stream);

/* (v, s) <- merge((v, s), (v_other, s_other)), in place. */
int rp_merge_state_in_place(void *v, float *s, const void *v_other, const float *s_other,
                            int64_t rows, int num_heads, int head_dim, void *stream);

/* Merge num_states (>= 1) states per row: v bf16 [rows][num_states][num_heads]
 * [head_dim], s fp32 [rows][num_states][num_heads] -> v_out bf16 [rows]
 * [num_heads][head_dim], s_out fp32 [rows][num_heads] (may be NULL). */
int rp_merge_states(const void *v, const float *s, void *v_out, float *s_out, int64_t rows,
                    int num_states, int num_heads, int head_dim, void *stream);

/* Shared-prefix attention (cascade attention over a two-level KV cache, page
 * "flashinfer-ai/flashinfer", cascade API, Cascade Attention; hierarchical KV
 * for shared prefixes, its feature list): every request of the batch attends
 * to the same shared_kv_len keys first, then to its own keys
 * kv_indptr[b]..kv_indptr[b+1].  The result equals attention over the
 * concatenation [shared keys, own keys] (with the causal mask, bottom-right
 * aligned, over that concatenation), up to rounding: it is computed as
 *   1. all query rows q_indptr[0]..q_indptr[batch] against the shared keys
 *      (one request, no mask) -> a bf16/fp32 state in the workspace,
 *   2. the ragged batch against the own keys (as rp_run) -> o,
 *   3. o, lse <- merge of the two states (rp_merge_state), in place.
 * So the shared K/V are read for all requests at once rather than once per
 * request, and the intermediate state is rounded to bf16 before the merge.
 * causal requires qo_len <= kv_len (own keys) in every request when
 * shared_kv_len > 0 (so that every row sees the whole prefix), else
 * RP_EINVAL.  The plan is used with rp_run_shared_prefix only (rp_run and
 * rp_run_paged reject it); rp_plan_get_info reports both levels (flops,
 * items; bytes add the shared K/V once) and rp_plan_workspace_bytes the whole
 * workspace. */
int rp_plan_create_shared_prefix(const int32_t *q_indptr, const int32_t *kv_indptr, int batch,
                                 int shared_kv_len, int num_qo_heads, int num_kv_heads,
                                 int head_dim, int causal, const rp_plan_opts *opts,
                                 rp_plan **out);

/* Run a shared-prefix plan.  k_shared, v_shared: bf16 [shared_kv_len]
 * [num_kv_heads][head_dim]; k_unique, v_unique: bf16 ragged per kv_indptr;
 * q, o, lse as for rp_run (lse may be NULL).  workspace: at least
 * rp_plan_workspace_bytes(plan) bytes, 256-byte aligned (never NULL: it holds
 * the shared-level state). */
int rp_run_shared_prefix(const rp_plan *plan, const void *q, const void *k_shared,
                         const void *v_shared, const void *k_unique, const void *v_unique,
                         void *o, float *lse, float sm_scale, void *workspace,
                         size_t workspace_bytes, void *stream);

/* rp_run_shared_prefix with each request's own keys in a paged cache (the
 * serving layout of the cascade: page "flashinfer-ai/flashinfer", cascade
 * API, shared-prefix batch decode/prefill over a paged KV cache): k_pages,
 * v_pages bf16 [num_pages][page_size][num_kv_heads][head_dim], block_table,
 * max_blocks_per_seq and page_size as for rp_run_paged (key j of request b
 * at page block_table[b * max_blocks_per_seq + j / page_size], slot
 * j % page_size).  The shared prefix stays one contiguous bf16 block, read
 * once for all requests; everything else as for rp_run_shared_prefix.  The
 * result is bit-identical to rp_run_shared_prefix on the same keys. */
int rp_run_shared_prefix_paged(const rp_plan *plan, const void *q, const void *k_shared,
                               const void *v_shared, const void *k_pages, const void *v_pages,
                               const int32_t *block_table, int max_blocks_per_seq, int page_size,
                               void *o, float *lse, float sm_scale, void *workspace,
                               size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RAGGED_PREFILL_H */
