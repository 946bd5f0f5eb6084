/*
 * bsp.h — C ABI of libbsp: one decode step of cascade attention for wide beam
 * search over a shared prompt, on a paged KV cache, for AMD MI355X (gfx950).
 *
 * The method (TensorRT-LLM PR #21738, "Add opt-in cascade attention for wide
 * beam search on KVCM V2", Description: Problem and Solution): all beams of a
 * request share one prompt, so the prompt's keys are attended once per request
 * with every beam's query rows at once, each beam's own generated tail is
 * attended separately through cache_indirection, and the two partial results
 * are merged exactly through their log-sum-exp. A beam-1 variant bounds the
 * key range to the valid cached prefix rounded up to 256 rows (Phi-4 cached-
 * prefix PR, TensorRT-Model-Connect #2202: Exit Criteria, Implementation).
 * Steps that also carry context requests (PR #21738, mixed-batches commit)
 * run those through a ragged causal prefill (bsp_plan_prefill,
 * bsp_prefill_attn) beside the beam step of the generation requests.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Device pointers belong to the caller. The library never allocates device
 *   memory; its only allocation is the pinned host staging owned by a plan.
 * - Every call is asynchronous and ordered on the caller's stream. Only
 *   bsp_check and check mode (environment BSP_CHECK=1 when the plan is
 *   created) wait for the device.
 * - Errors: each call returns a bsp_status_t; bsp_last_error() gives a
 *   message for the calling thread. A call that fails validation returns
 *   before any launch and leaves every buffer unchanged. Indices are never
 *   clamped (the eligibility commit of PR #21738 raises on a bad prompt page
 *   index rather than clamping it).
 * - Index values that only the device sees (slots, cache_indirection entries,
 *   device block-table entries) are bounds-checked in the kernels: a bad one
 *   is skipped and recorded in the plan workspace's error word, which
 *   bsp_check reports.
 * - Layouts (all row-major, innermost last):
 *     K/V pool        [num_pages, num_kv_heads, page_size, head_dim]
 *     q               [B, W, q_len, num_q_heads, head_dim]
 *     block tables    int32 [B, W, max_blocks_per_seq]
 *     cache_indirection int32 [B, W, max_seq_len]
 *     partial o       float [n_parts][B * W * q_len][num_q_heads][head_dim]
 *     partial lse     float [n_parts][B * W * q_len][num_q_heads]
 *     prefill q / o   [sum of chunk rows][num_q_heads][head_dim], request-major
 *   Query head h reads KV head h / (num_q_heads / num_kv_heads).
 * - LSE is the natural log of the softmax denominator, scale included; an
 *   empty key set gives o = 0 and lse = -inf.
 */
#ifndef BSP_H
#define BSP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { BSP_F32 = 0, BSP_F16 = 1, BSP_BF16 = 2 } bsp_dtype_t;

/* Self mask of the query rows when q_len > 1. */
typedef enum {
  BSP_MASK_NONE = 0,   /* every query row sees every valid key                 */
  BSP_MASK_CAUSAL = 1  /* row i of q_len sees keys j <= n_keys - q_len + i     */
} bsp_mask_t;

typedef enum {
  BSP_OK = 0,
  BSP_ERR_ARG = 1,            /* null pointer, bad size, misaligned buffer        */
  BSP_ERR_PAGE_INDEX = 2,     /* a host block-table entry outside [0, num_pages)  */
  BSP_ERR_TAIL_OVERFLOW = 3,  /* a tail longer than the fixed max_tail            */
  BSP_ERR_DTYPE = 4,          /* unsupported dtype                                 */
  BSP_ERR_UNSUPPORTED = 5,    /* unsupported geometry (head_dim, page_size, ...)  */
  BSP_ERR_STALE_PLAN = 6,     /* attention call on a plan with no bsp_plan yet    */
  BSP_ERR_WORKSPACE = 7,      /* workspace missing or too small                    */
  BSP_ERR_DEVICE_INDEX = 8,   /* a kernel met an out-of-range index (bsp_check)   */
  BSP_ERR_HIP = 9             /* a HIP runtime call failed                          */
} bsp_status_t;

/* Geometry of one attention layer. */
typedef struct {
  int32_t num_q_heads;    /* Hq, a multiple of num_kv_heads                          */
  int32_t num_kv_heads;   /* Hkv                                                      */
  int32_t head_dim;       /* D: 64, 128 or 256                                        */
  int32_t page_size;      /* rows per page: a power of two, 1..1024                   */
  int32_t num_pages;      /* pages in each of the K and V pools                       */
  int32_t dtype;          /* bsp_dtype_t of q, the pools and the final output         */
  float sm_scale;         /* softmax scale; 0 selects 1/sqrt(head_dim)                */
  int32_t max_tail;       /* 0: tail length set per step; > 0: fixed padded tail
                             length (graph-style), a longer tail is an error
                             (PR #21738: Correctness and limits; MAX_TAIL thread)     */
  int32_t key_bucket;     /* 0: beam mode, the shared keys are the prompt rows;
                             > 0: cached-prefix mode, rows bound per request =
                             valid rows rounded up to key_bucket, capped at
                             max_cache_rows, 1 for an empty cache (PR #2202)           */
  int32_t max_cache_rows; /* cap of the bound rows in cached-prefix mode              */
  int32_t mask;           /* bsp_mask_t of the query rows (q_len > 1)                 */
  int32_t kv_split;       /* 0: one pass over the shared keys; > 0: split them into
                             chunks of this many keys (a multiple of 64), each
                             giving its own partial (o, lse) to merge afterwards;
                             -1: bsp_plan picks the chunk per step, the smallest
                             multiple of 64 keys whose work items (request, KV
                             head, chunk, query tile) fit one round of 512
                             workgroups (two per CU), no split if none is smaller
                             than the longest key range (bsp_prefix_attn only)      */
} bsp_layer_desc_t;

typedef struct bsp_plan_s* bsp_plan_t;

/* bsp_plan_create flags */
#define BSP_PLAN_HOST_ONLY 1u /* validation and table building only: no HIP calls,
                                 bsp_plan must get a null workspace, and only the
                                 bsp_debug_* host getters may follow              */

/* Thread-local message of the last failed call on this thread ("" if none). */
const char* bsp_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int32_t bsp_version(void);

/*
 * Create a per-step plan object for one layer geometry and its capacity. The
 * plan is made once per step and read by every layer of that step (PR #21738,
 * first commit: the host plan runs once per step before graph capture or
 * replay). It owns two pinned host staging buffers and nothing on the device.
 * Errors: BSP_ERR_ARG, BSP_ERR_UNSUPPORTED, BSP_ERR_DTYPE, BSP_ERR_HIP.
 */
bsp_status_t bsp_plan_create(const bsp_layer_desc_t* desc, int32_t max_requests,
                             int32_t max_beam, int32_t max_blocks_per_seq,
                             int32_t max_seq_len, int32_t max_q_len, uint32_t flags,
                             bsp_plan_t* out);

/* Bytes of device workspace the caller must provide to bsp_plan (256-aligned,
 * caller-owned; zero-filled once after allocation). 0 on a null plan. */
size_t bsp_plan_workspace_bytes(bsp_plan_t plan);

/* Destroy a plan (waits for its in-flight staging copies). Null is a no-op. */
void bsp_plan_destroy(bsp_plan_t plan);

/*
 * Plan one step: validate lengths and page ids on the host, build the shared-
 * key page table of each request from beam 0's block table (PR #21738, KV-
 * cache-manager-V2 commit: the prompt page table is beam 0's), the tail
 * lengths and the key bounds, and copy them into workspace_d with an
 * asynchronous copy from pinned staging on `stream`, without waiting for the
 * stream (PR #21738, commit making re-planning non-blocking).
 *
 *   B, W, q_len          requests, beams per request, query rows per beam
 *   prefix_len_h[B]      beam mode: prompt rows shared by the W beams (P_b);
 *                        cached-prefix mode: valid cached rows (L_b)
 *   seq_len_h[B]         beam mode: cached rows of each beam, P_b + tail (S_b);
 *                        cached-prefix mode: must equal prefix_len_h
 *   block_tables_h       host copy of the block tables, int32 [B][W][max_blocks]
 *   workspace_d          caller device buffer of bsp_plan_workspace_bytes bytes
 *                        (null for a BSP_PLAN_HOST_ONLY plan)
 * Checks: 0 <= P_b <= S_b <= max_seq_len; tail <= max_tail when max_tail > 0
 * (BSP_ERR_TAIL_OVERFLOW); every block-table entry the step reads (beam 0's
 * shared blocks, every beam's tail blocks) in [0, num_pages)
 * (BSP_ERR_PAGE_INDEX); in check mode, also that all beams share the full
 * prompt blocks. On failure the previous plan is dropped (BSP_ERR_STALE_PLAN
 * until the next successful call).
 */
bsp_status_t bsp_plan(bsp_plan_t plan, int32_t B, int32_t W, int32_t q_len,
                      const int32_t* prefix_len_h, const int32_t* seq_len_h,
                      const int32_t* block_tables_h, void* workspace_d,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * bsp_plan without a caller workspace, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that forbid
 * allocation): the plan's tables go into a static scratch array the library
 * holds on each device it runs on (32 MiB, kept until the process ends; its
 * address is looked up once per device on the first call there). Arguments,
 * checks and the non-blocking copy are those of bsp_plan; every later call of
 * the plan (bsp_decode_step, bsp_prefix_attn, ...) uses that scratch. The call
 * allocates nothing. A plan whose bsp_plan_workspace_bytes exceeds 32 MiB is
 * rejected with BSP_ERR_WORKSPACE. All plans planned this way on one device
 * share its array, which keeps the last call's contents (each call rewrites
 * everything a step reads, error word and split counters included): calls,
 * and the steps that read their plans, that overlap on one device race, so
 * order them on one stream and use one such plan at a time per device.
 */
bsp_status_t bsp_plan_static(bsp_plan_t plan, int32_t B, int32_t W, int32_t q_len,
                             const int32_t* prefix_len_h, const int32_t* seq_len_h,
                             const int32_t* block_tables_h, hipStream_t stream);

/* Number of partial states bsp_prefix_attn writes for the current plan (1 when
 * kv_split is 0), the keys per split (0: one pass; the chosen chunk when
 * kv_split is -1), and the tail length each beam is padded to. -1 if
 * unplanned. */
int32_t bsp_plan_num_splits(bsp_plan_t plan);
int32_t bsp_plan_split_keys(bsp_plan_t plan);
int32_t bsp_plan_tail_len(bsp_plan_t plan);

/*
 * Write n new tokens' K and V rows into the pools: token i goes to page
 * slots[i] / page_size, row slots[i] % page_size, for all KV heads, K and V in
 * one launch (TensorRT-LLM PR #18614, Description: one launch derives page and
 * row from the flat slot and writes K and V together).
 *   k_new, v_new   device, token i's [num_kv_heads, head_dim] block starts at
 *                  element i * src_row_stride (16-byte aligned)
 *   slots_d        device int32 [n]; a slot outside [0, num_pages*page_size)
 *                  is skipped and recorded in the error word
 * n == 0 succeeds without a launch. Uses the plan's geometry and workspace
 * (bsp_check reports skipped slots), so the plan must have been planned once.
 */
bsp_status_t bsp_write_kv(bsp_plan_t plan, const void* k_new, const void* v_new,
                          int64_t src_row_stride, const int32_t* slots_d, int32_t n,
                          void* k_pool, void* v_pool, hipStream_t stream);

/*
 * bsp_write_kv from the layer descriptor alone, with no plan: the same write
 * (TensorRT-LLM PR #18614, Description: page and row from the flat slot, K and
 * V in one launch) for callers that write a token before, or without, a step
 * plan. The descriptor is checked as bsp_plan_create checks it (dtype,
 * num_kv_heads, head_dim, page_size, num_pages; the other fields are not
 * used). Skipped slots are counted in faults_d, device int32[3] or null:
 * [0] becomes nonzero (an OR of error bits), [1] counts the skipped tokens and
 * [2] holds one skipped slot value; the caller zeroes it, the call never does.
 * With faults_d null, skipped slots leave no trace. Asynchronous on `stream`;
 * n == 0 succeeds without a launch.
 */
bsp_status_t bsp_write_kv_desc(const bsp_layer_desc_t* desc, const void* k_new, const void* v_new,
                               int64_t src_row_stride, const int32_t* slots_d, int32_t n,
                               void* k_pool, void* v_pool, int32_t* faults_d, hipStream_t stream);

/*
 * Shared-key attention: for each request b and KV head g, all W * q_len * G
 * query rows (G = num_q_heads / num_kv_heads) against the request's shared
 * keys, once per request (PR #21738, Solution: the prompt is attended once per
 * request; FA4 commit: one group of beam_width queries per request). Keys are
 * rows [0, valid_b) of the request's page table; in cached-prefix mode rows in
 * [valid_b, bound_b) are masked and rows past the bound are never read.
 * Writes bsp_plan_num_splits() normalised partial states: o_part (float,
 * [n_split][B*W*q_len][Hq][D]) and lse_part (float, [n_split][B*W*q_len][Hq]).
 * bf16/f16 run on MFMA; f32 runs a vector-ALU kernel.
 */
bsp_status_t bsp_prefix_attn(bsp_plan_t plan, const void* q, const void* k_pool,
                             const void* v_pool, float* o_part, float* lse_part,
                             hipStream_t stream);

/*
 * bsp_prefix_attn for two plans of the same layer and query rows in one
 * launch: plan a writes o_part_a / lse_part_a, plan b writes o_part_b /
 * lse_part_b, exactly as two bsp_prefix_attn calls would. For the two key
 * segments of one masked cached-prefix call (PR #2202, Implementation: the
 * cached rows up to the bound, then this call's rows), whose partials are
 * then merged with bsp_merge. Both plans must be planned, with the same
 * dtype, head counts, head_dim and B * W * q_len; q and the pools are shared.
 * When both plans take one 64-row query tile per work item (bf16/f16) the
 * work of both runs in one launch; otherwise the call makes one launch per
 * plan. Errors as for bsp_prefix_attn, checked for both plans before any
 * launch.
 */
bsp_status_t bsp_prefix_attn_two(bsp_plan_t a, bsp_plan_t b, const void* q, const void* k_pool,
                                 const void* v_pool, float* o_part_a, float* lse_part_a,
                                 float* o_part_b, float* lse_part_b, hipStream_t stream);

/*
 * A whole one-row cached-prefix decode call in one launch (PR #2202,
 * Background and Implementation: a decode step attends the valid cached rows,
 * bounded to the bucket, plus its own row; TensorRT-LLM PR #21738, review
 * thread on the FA4 split-generation kernels: split the keys, then merge the
 * splits). The plan (key_bucket > 0, W = 1, q_len = 1, at most 64 query rows
 * per KV head, bf16/f16) splits the valid cached rows into chunks
 * (bsp_plan_num_splits); each chunk's workgroup writes its partial state to
 * o_part/lse_part (as bsp_prefix_attn) and counts itself on a counter in the
 * workspace; the last chunk of each (request, KV head) to finish merges all
 * chunks, in chunk order, with this call's row -- its key and value read from
 * k_new/v_new, visible to the row itself -- into o_out (dtype [B][Hq][D]) and
 * lse_out (float [B][Hq], may be null), and writes the new row into the pools
 * at slots_d[b] (device int32 [B], page * page_size + row; a slot outside the
 * pool is skipped and recorded for bsp_check). No workgroup waits for another.
 *   q             [B, 1, 1, Hq, D]
 *   k_new, v_new  request b's new row at element b * new_row_stride, [Hkv][D]
 *   o_part        float [n_split][B][Hq][D]; lse_part float [n_split][B][Hq]
 * The same result as bsp_write_kv + bsp_prefix_attn (cache) + bsp_prefix_attn
 * (the new row) + bsp_merge, up to fp32 summation order. The counters live in
 * the plan's workspace and each last chunk resets its own, so launches of one
 * plan must be ordered (one stream); overlapping launches of one plan race.
 * Errors as for bsp_prefix_attn, and BSP_ERR_UNSUPPORTED for other plans, for
 * (Hq / Hkv) * D / 4 > 256, and for partial states of more than 4 GiB
 * (n_split * B * Hq * D * 4 bytes: the merge addresses them with 32-bit offsets).
 */
bsp_status_t bsp_cached_decode(bsp_plan_t plan, const void* q, const void* k_new, const void* v_new,
                               int64_t new_row_stride, const int32_t* slots_d, void* k_pool,
                               void* v_pool, float* o_part, float* lse_part, void* o_out,
                               float* lse_out, hipStream_t stream);

/*
 * The one-row cached-prefix decode in two launches: bsp_prefix_attn on the
 * plan (the cache chunks' partial states into o_part/lse_part), then this
 * call, which merges them exactly with the call's own row (PR #2202,
 * Background: a decode step attends the valid cached rows plus its own row;
 * TensorRT-LLM PR #21738, Description: Solution, merged with the log-sum-exp)
 * -- the row is one more part, its score scale * q . k_new and its value
 * v_new -- into o_out (dtype [B][Hq][D]) and lse_out (float [B][Hq], may be
 * null), and writes the row into the pools at slots_d[b] (device int32 [B],
 * page * page_size + row; a slot outside the pool is skipped and recorded for
 * bsp_check). No separate KV write is needed, and the new row is never read
 * from the pool.
 *   q             [B, 1, 1, Hq, D]
 *   k_new, v_new  request b's new row at element b * new_row_stride, [Hkv][D],
 *                 16-byte aligned; new_row_stride a multiple of 8
 *   o_part        float [n_split][B][Hq][D], 16-byte aligned; lse_part float
 *                 [n_split][B][Hq], as bsp_prefix_attn wrote them for this plan
 * The same result as bsp_cached_decode, up to fp32 summation order. The plan
 * as for bsp_cached_decode (key_bucket > 0, W = 1, q_len = 1, bf16/f16):
 * BSP_ERR_UNSUPPORTED otherwise; BSP_ERR_ARG for null or misaligned pointers.
 */
bsp_status_t bsp_cached_decode_merge(bsp_plan_t plan, const void* q, const void* k_new,
                                     const void* v_new, int64_t new_row_stride,
                                     const int32_t* slots_d, void* k_pool, void* v_pool,
                                     const float* o_part, const float* lse_part, void* o_out,
                                     float* lse_out, hipStream_t stream);

/*
 * Tail attention: each beam's G query rows against its own tail positions
 * P_b <= j < S_b, gathered through cache_indirection: position j of beam k is
 * read from beam src = cache_indirection[b][k][j], page
 * block_tables[b][src][j / page_size], row j % page_size (PR #21738, Solution
 * and fused-tail commit). q_len must be 1. Writes o_tail (float,
 * [B*W][Hq][D]) and lse_tail (float, [B*W][Hq]); an empty tail gives o = 0,
 * lse = -inf.
 *   block_tables_d      device int32 [B][W][max_blocks_per_seq]
 *   cache_indirection_d device int32 [B][W][max_seq_len]
 */
bsp_status_t bsp_tail_attn(bsp_plan_t plan, const void* q, const void* k_pool,
                           const void* v_pool, const int32_t* block_tables_d,
                           const int32_t* cache_indirection_d, float* o_tail,
                           float* lse_tail, hipStream_t stream);

/*
 * Exact merge of n_parts partial states over disjoint key sets (PR #21738,
 * Solution: merged exactly with the log-sum-exp):
 *   lse = ln sum_p exp(lse_p),  o = sum_p exp(lse_p - lse) * o_p.
 * Parts with lse = -inf drop out; all empty gives o = 0, lse = -inf.
 *   o_parts   float, part p at o_parts + p * o_part_stride, [rows][heads][head_dim]
 *   lse_parts float, part p at lse_parts + p * lse_part_stride, [rows][heads]
 *   o_out     out_dtype [rows][heads][head_dim]; lse_out float [rows][heads] or null
 */
bsp_status_t bsp_merge(int32_t rows, int32_t heads, int32_t head_dim, int32_t n_parts,
                       const float* o_parts, const float* lse_parts, int64_t o_part_stride,
                       int64_t lse_part_stride, void* o_out, int32_t out_dtype,
                       float* lse_out, hipStream_t stream);

/*
 * The whole beam decode step of one layer in one launch (the fused form of
 * bsp_write_kv + bsp_prefix_attn + bsp_tail_attn + bsp_merge; PR #21738,
 * fused-tail commit: the current-token KV write, the tail attention through
 * cache_indirection and the merge with the prefix run as one launch per
 * layer). For each request and KV head one workgroup writes its beams'
 * current tokens into their pages, attends every beam's query rows to the
 * shared prompt and then to the beam's own tail in the same online softmax
 * (so the merge is exact and no partial state leaves the kernel), and writes
 * the final output. The tail position S_b - 1 (the current token) is read from
 * k_new/v_new of the parent beam, never from the pool being written.
 *   q              [B, W, 1, Hq, D] (plan q_len must be 1; beam mode; no kv_split)
 *   k_new, v_new   current token of every beam: row (b * W + k) at element
 *                  (b * W + k) * new_row_stride, [Hkv][D] contiguous, 16-byte
 *                  aligned; rows of requests without a tail are not read
 *   k_pool, v_pool written at each beam's slot for position S_b - 1
 *   o_out          dtype [B * W][Hq][D], 16-byte aligned; lse_out float
 *                  [B * W][Hq] or null
 * q and the pools are 16-byte aligned too (BSP_ERR_ARG otherwise).
 * bf16/f16 only (BSP_ERR_UNSUPPORTED for f32: use the separate calls).
 * Work items go longest first (when they fill more than one round of
 * workgroups, a request's W x tail rows count as keys; in one round the
 * shorter half is listed shortest first). When the plan split a request's
 * prompt into chunks (see bsp_debug_plan_items), each chunk's workgroup leaves its partial
 * state in the workspace and counts itself with one atomic add; the last to
 * arrive merges the states exactly through their log-sum-exp (PR #21738,
 * Solution) and finishes the request. No workgroup waits for another. Calls
 * that share one workspace must be ordered on one stream (as for every call
 * of a plan).
 */
bsp_status_t bsp_decode_step(bsp_plan_t plan, const void* q, const void* k_new,
                             const void* v_new, int64_t new_row_stride, void* k_pool,
                             void* v_pool, const int32_t* block_tables_d,
                             const int32_t* cache_indirection_d, void* o_out, float* lse_out,
                             hipStream_t stream);

/*
 * Context phase of a mixed step (PR #21738, mixed-batches commit: a step may
 * carry context requests ahead of the generation requests; the library serves
 * the generation rows and the context rows go through a regular paged causal
 * prefill). Plans C context requests of one chunk each: request b has
 * cached_len_h[b] = L_b rows already in its pages and q_len_h[b] = Sq_b new
 * rows (1 <= Sq_b <= max_q_len, L_b + Sq_b <= max_seq_len), whose K/V the
 * caller writes at positions L_b .. L_b + Sq_b - 1 of the request's pages
 * (bsp_write_kv) before bsp_prefill_attn runs. block_tables_h: host int32
 * [C][max_blocks_per_seq], the first ceil((L_b + Sq_b) / page_size) entries of
 * each row read (BSP_ERR_PAGE_INDEX outside [0, num_pages)). Replaces the
 * plan's current step: the beam entry points reject a plan holding a prefill
 * step (BSP_ERR_ARG) until the next bsp_plan. Plans without key_bucket only.
 * Workspace, staging and stream rules as for bsp_plan.
 */
bsp_status_t bsp_plan_prefill(bsp_plan_t plan, int32_t C, const int32_t* q_len_h,
                              const int32_t* cached_len_h, const int32_t* block_tables_h,
                              void* workspace_d, size_t workspace_bytes, hipStream_t stream);

/*
 * Causal paged attention of the planned context requests: query row i of
 * request b (packed row q_off_b + i, q_off_b = Sq_0 + ... + Sq_{b-1}) attends
 * the request's keys 0 .. L_b + i (its cached rows and the chunk's rows up to
 * its own), query head h reading KV head h / G. One launch for the whole
 * ragged batch.
 *   q        dtype [sum Sq_b][Hq][D], 16-byte aligned
 *   k_pool, v_pool  as for bsp_prefix_attn, holding the chunk's rows already
 *   o_out    dtype [sum Sq_b][Hq][D]; lse_out float [sum Sq_b][Hq] or null
 * bf16/f16 only (BSP_ERR_UNSUPPORTED for f32). BSP_ERR_STALE_PLAN without a
 * prefill step. Out-of-range page ids met on the device are skipped and
 * recorded for bsp_check.
 */
bsp_status_t bsp_prefill_attn(bsp_plan_t plan, const void* q, const void* k_pool,
                              const void* v_pool, void* o_out, float* lse_out,
                              hipStream_t stream);

/*
 * A whole mixed step of one layer (PR #21738, mixed-batches commit): the beam
 * step of the generation requests (`gen`, planned by bsp_plan; the arguments of
 * bsp_decode_step) and the causal prefill of the context requests (`ctx`,
 * planned by bsp_plan_prefill; the arguments of bsp_prefill_attn, whose chunk
 * rows the caller has written with bsp_write_kv on this stream before). The
 * two parts touch disjoint rows and may share one pool (pass it twice). When
 * both parts take one 16-row query block per wave (the beam step's W * G <= 64
 * rows per request, the prefill plan's 64-row items), head_dim <= 128, the
 * beam step's tails fit its slot table and it has no balanced pairs, this is
 * one launch in which beam-step and context workgroups share the CUs (the
 * first bandwidth-bound, the second latency- and matrix-bound); otherwise the
 * prefill, then the beam step, on the stream. Results and errors as for the
 * two calls; the plans must have the same dtype and head_dim.
 */
bsp_status_t bsp_mixed_step(bsp_plan_t gen, bsp_plan_t ctx, const void* q, const void* k_new,
                            const void* v_new, int64_t new_row_stride, void* k_pool, void* v_pool,
                            const int32_t* block_tables_d, const int32_t* cache_indirection_d,
                            void* o_out, float* lse_out, const void* q_ctx, const void* k_pool_ctx,
                            const void* v_pool_ctx, void* o_ctx, float* lse_ctx,
                            hipStream_t stream);

/*
 * Comparator, not part of the cascade: per-beam attention over each beam's
 * whole sequence, reading the shared prompt once per (beam, KV head) through
 * the beam's own block table, as the decode kernel that the cascade replaces
 * does (PR #21738, first commit: the legacy kernel re-reads the prompt KV once
 * per beam and head). Final output o_out (dtype, [B*W][Hq][D]) and lse_out
 * (float, [B*W][Hq], may be null). q_len must be 1.
 */
bsp_status_t bsp_naive_beam_attn(bsp_plan_t plan, const void* q, const void* k_pool,
                                 const void* v_pool, const int32_t* block_tables_d,
                                 const int32_t* cache_indirection_d, void* o_out,
                                 float* lse_out, hipStream_t stream);

/* Wait for `stream`, then report (and clear) any index fault the kernels
 * recorded in the plan's workspace: BSP_ERR_DEVICE_INDEX with a message. */
bsp_status_t bsp_check(bsp_plan_t plan, hipStream_t stream);

/* Test hooks -------------------------------------------------------------- */

/* Host copy of the current plan's tables (valid for host-only plans too):
 * indptr[B+1], pages[indptr[B]], and per request n_keys (rows the page table
 * covers), valid (attended rows) and tail length. Any pointer may be null. */
bsp_status_t bsp_debug_plan_tables(bsp_plan_t plan, int32_t* indptr_h, int32_t* pages_h,
                                   int32_t* n_keys_h, int32_t* valid_h, int32_t* tail_h);

/* Host copy of the current plan's work items of bsp_decode_step (beam decode,
 * bf16/f16), in the order the step dispatches them (longest first):
 * *n_items_h, and when items_h is not null, int32 [n_items][4] = (request,
 * first key, end key, chunks of that request). A request whose prompt the
 * plan split has one item per chunk (TensorRT-LLM PR #21738, review thread on
 * the FA4 split-generation kernels: split the keys, then merge the splits).
 * By default bsp_plan splits when its model of the step (items dealt longest
 * first to one round of workgroups) gets at least 5% shorter;
 * BSP_SPLIT=<keys> in the environment at bsp_plan_create forces chunks of
 * that many keys (rounded up to 64) and BSP_SPLIT=0 turns splitting off. */
bsp_status_t bsp_debug_plan_items(bsp_plan_t plan, int32_t* n_items_h, int32_t* items_h);

/* Device: resolve every tail key to its flat pool slot (page * page_size +
 * row), int32 [B][W][tail_len], -1 past each request's tail; the same index
 * path bsp_tail_attn reads through. */
bsp_status_t bsp_debug_tail_slots(bsp_plan_t plan, const int32_t* block_tables_d,
                                  const int32_t* cache_indirection_d, int32_t* slots_d,
                                  hipStream_t stream);

/* Device: bsp_decode_step's own tail-slot table (TensorRT-LLM PR #21738,
 * Solution: each beam's tail is gathered through cache_indirection), as the
 * fused kernel builds it in LDS, written out instead of being used. The launch
 * runs the step with the same arguments as bsp_decode_step up to the point
 * where the table is complete (after the prompt, and after the merge of a
 * split request), writes it and stops: no tails, no output, no token write
 * (o_out is not written; the pools are only read). Entry (b, g, beam, t), for
 * KV head g and tail position t < S_b - P_b, is written at int32
 * slots_out_d[((b * Hkv + g) * W + beam) * max(tail_len, 1) + t] (tail_len =
 * bsp_plan_tail_len); other entries are left as they were. An entry >= 0 is
 * the pool row ((page * Hkv + g) * page_size + row); an entry <= -2 is the
 * current token, read from the new-token row of beam (-entry - 2); -1 an
 * invalid index (also recorded for bsp_check). BSP_ERR_UNSUPPORTED where the
 * step gathers the tails key by key (tails too long for the LDS table). */
bsp_status_t bsp_debug_fused_slots(bsp_plan_t plan, const void* q, const void* k_new,
                                   const void* v_new, int64_t new_row_stride, void* k_pool,
                                   void* v_pool, const int32_t* block_tables_d,
                                   const int32_t* cache_indirection_d, void* o_out,
                                   int32_t* slots_out_d, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BSP_H */
