// Internal declarations shared by the host planner (bsp_host.cpp) and the HIP
// kernels. Not part of the public ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/bsp.h"

namespace bsp {

// ---------------------------------------------------------------------------
// Device workspace written by bsp_plan (caller-owned device memory).
//
//   [0, 256)                 header: error word, fault count, first bad value
//   [256, 256 + 32*maxB)     per-request info, ReqInfo
//   then                     shared-key page table, int32 [sum of pages]
// ---------------------------------------------------------------------------
constexpr size_t kHeaderBytes = 256;

enum ErrorBits : int32_t {
  kErrPrefixPage = 1,   // a shared-key page id outside [0, num_pages)
  kErrTailParent = 2,   // a cache_indirection entry outside [0, W)
  kErrTailPage = 4,     // a tail block-table entry outside [0, num_pages)
  kErrWriteSlot = 8,    // a KV-write slot outside [0, num_pages * page_size)
};

struct DevHeader {
  int32_t error_bits;   // OR of ErrorBits
  int32_t fault_count;
  int32_t first_value;  // the first offending value a kernel saw (racy, informative)
  int32_t pad[61];
};
static_assert(sizeof(DevHeader) == kHeaderBytes, "header size");

// Per-thread floats of one partial state of the fused step (a request's prompt
// split over several workgroups): O accumulators (D/16 blocks x MB query
// blocks x 4), then the running max and sum per query block; stored
// element-major over the 256 threads of a workgroup, so that the workgroup
// that merges reads back exactly the elements each of its threads holds.
constexpr int split_part_floats(int head_dim, int mb) { return (head_dim / 16) * mb * 4 + 2 * mb; }
// Device bytes the plan reserves for split partial states at most.
constexpr size_t kSplitPartBudget = size_t(24) << 20;

struct ReqInfo {
  int32_t page_off;  // first entry of this request in the page table
  int32_t n_keys;    // rows the page table covers (P_b, or the bound rows)
  int32_t valid;     // rows attended (P_b, or the valid cached rows L_b)
  int32_t prefix;    // P_b
  int32_t seq;       // S_b
  int32_t tail;      // S_b - P_b
  int32_t n_split;   // splits holding keys
  int32_t q_off;     // prefill plans: first packed query row of this request (else 0)
};
// In prefill plans (bsp_plan_prefill) prefix = L_b cached rows before the
// chunk, tail = the chunk's rows (the query rows), seq = n_keys = valid = L_b +
// chunk rows: the page table covers the cached rows and the chunk's own rows.
static_assert(sizeof(ReqInfo) == 32, "ReqInfo size");

// One work item of the fused step: keys [k_lo, k_hi) of request b's prompt
// (all of it unless the plan split the prompt). Items are listed longest
// first, so the workgroups that stream the most keys are dispatched first.
// A split request's `parts` items each leave a partial state in slots
// [slot, slot + parts) and count themselves on the request's counter; the
// last to arrive merges the others and finishes the request (tails, output,
// current-token write). Unsplit: parts = 1, slot = -1.
struct FusedItem {
  ReqInfo ri;        // request b's info, copied so that one load gives a workgroup its work
  int32_t b, k_lo, k_hi, part;
  int32_t parts, slot, pad0, pad1;
};
static_assert(sizeof(FusedItem) == 64, "FusedItem size");

// ---------------------------------------------------------------------------
// Kernel parameter blocks (passed by value).
// ---------------------------------------------------------------------------
struct WriteKvParams {
  const void* k_new;
  const void* v_new;
  int64_t src_stride;   // elements between consecutive tokens
  const int32_t* slots;
  int32_t n;
  void* k_pool;
  void* v_pool;
  int32_t hkv, d, page_size;
  int64_t num_slots;
  int32_t* fault;       // device int32[3] (error bits, fault count, first value) or null
};

struct PrefixParams {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  float* o_part;
  float* lse_part;
  const ReqInfo* req;
  // fused step: its work items, longest first (blocks are dispatched in order)
  const FusedItem* fitems;
  const int32_t* pages;
  DevHeader* hdr;
  int32_t B, W, q_len, hq, hkv, group;
  int32_t page_shift;   // log2(page_size)
  int32_t num_pages;
  int32_t n_split, split_keys, n_qtiles;
  // 1: the query tiles of one work item take block ids 8 apart (one XCD, one
  // L2 for the keys they all read); needs B * hkv * n_split % 8 == 0
  int32_t xcd_remap;
  int32_t causal;
  int32_t rows_total;   // B * W * q_len (prefill: packed rows)
  const int32_t* items; // prefill: work list, (request, query tile) int32 pairs
  float scale;          // softmax scale
  float scale_log2e;    // scale * log2(e)
};

// Extra inputs of the fused decode step (prefix + tail + current-token write
// in one launch; q_len 1, beam mode).
struct FusedParams {
  const void* k_new;            // current token of every beam, [B*W][Hkv*D] with row stride
  const void* v_new;
  int64_t new_stride;           // elements between consecutive beams' rows
  void* k_pool_w;               // the pools again, writable (the token write)
  void* v_pool_w;
  const int32_t* block_tables;  // device [B][W][max_blocks]
  const int32_t* ci;            // device [B][W][max_seq_len]
  int32_t max_blocks, max_seq_len;
  void* o_out;                  // dtype [B*W][Hq][D]
  float* lse_out;               // [B*W][Hq] or null
  // split requests (null when the plan split none): arrival counters
  // [B][Hkv][n_qtiles], zero between launches (the last arrival resets its
  // counter), and partial states [slot][Hkv][n_qtiles][part_floats][256]
  int32_t* split_count;
  float* split_part;
  int32_t part_floats;
  // one-launch cached-prefix decode (bsp_cached_decode, MODE 5): the chunks'
  // partial states are counted on split_count per (request, KV head), and the
  // last chunk to arrive merges them with the new row (k_new/v_new) into
  // o_out/lse_out and writes the new row at new_slots[b]
  const int32_t* new_slots;
  // debug (bsp_debug_fused_slots): when set, the beam step (MODE 1) writes its
  // LDS tail-slot table here, entry (b, g, beam, t) at
  // ((b * Hkv + g) * W + beam) * dump_pad + t, and stops before the tails
  int32_t* dump_slots;
  int32_t dump_pad;
  // the beam step's output and current-token rows go out with non-temporal
  // stores (set by the host when they fit the L2s, kStreamOutBytes)
  int32_t stream_out;
};

struct TailParams {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* ci;
  float* o_tail;
  float* lse_tail;
  int32_t* slots_out;   // debug: resolved slots [B*W*tail_pad] or null
  const ReqInfo* req;
  DevHeader* hdr;
  int32_t B, W, hq, hkv, group;
  int32_t page_shift, num_pages;
  int32_t max_blocks, max_seq_len, tail_pad;
  float scale, scale_log2e;
};

struct MergeParams {
  int32_t rows, heads, d, n_parts;
  const float* o_parts;
  const float* lse_parts;
  int64_t o_stride, lse_stride;
  void* o_out;
  float* lse_out;
};

// A beam step with one or two query blocks per wave whose output, LSE and
// current-token writes total at most this many bytes writes them with
// non-temporal stores: written normally they would all still be dirty in the
// eight XCDs' L2s (4 MB each) when the kernel ends, and the write-back there
// runs after the last workgroup. Larger writes drain during the kernel anyway,
// and the hint measured slightly slower there.
constexpr int64_t kStreamOutBytes = int64_t(24) << 20;
// Bytes of the library's static device scratch (bsp_plan_static).
constexpr size_t kStaticWorkspaceBytes = size_t(32) << 20;
// The calling thread's error message (bsp_last_error) and status.
bsp_status_t set_error(bsp_status_t st, const char* fmt, ...);
// Make the plan's next bsp_plan copy the whole workspace header again.
void forget_workspace(bsp_plan_t plan);

// ---------------------------------------------------------------------------
// Launchers (defined next to their kernels). They return hipSuccess or the
// launch error; shape checks are done by the host entry points beforehand.
// ---------------------------------------------------------------------------
hipError_t launch_write_kv(const WriteKvParams& p, int dtype, hipStream_t s);
// `rows_per_tile`: query rows per work item as the plan chose it (a multiple of 64
// on the matrix cores, prefix_rows_per_tile() or fewer).
hipError_t launch_prefix(const PrefixParams& p, int dtype, int head_dim, int rows_per_tile,
                         hipStream_t s);
// The cache chunks of a one-row cached-prefix decode and, in the last chunk of
// each (request, KV head) to finish, the merge with the new row (bf16/f16,
// one 64-row query tile per item).
hipError_t launch_cached_decode(const PrefixParams& p, const FusedParams& f, int dtype,
                                int head_dim, hipStream_t s);
// Whether the one-launch decode's merge takes this shape (query heads per KV
// head x head_dim / 4 at most 256).
bool cached_decode_supported(int group, int head_dim);
// Two plans' bsp_prefix_attn work in one launch; both take 64 query rows per
// work item (bf16/f16 only).
hipError_t launch_prefix_two(const PrefixParams& a, const PrefixParams& b, int dtype, int head_dim,
                             hipStream_t s);
hipError_t launch_decode_step(const PrefixParams& p, const FusedParams& f, int dtype,
                              int head_dim, int rows_per_req, int n_items, int tail_pad,
                              hipStream_t s);
// Whether bsp_decode_step resolves the tails through its LDS slot table (MODE 1)
// for this shape, rather than key by key (MODE 2).
bool decode_uses_slot_table(int head_dim, int rows_per_req, int W, int group, int tail_pad);
// Query-row blocks of 16 per wave for an M-row item (4 waves per workgroup).
// At head_dim 256 a 128-row tile needs more than half a SIMD's registers (one
// workgroup per CU); 64-row tiles at two per CU, the tiles of a request on one
// XCD, measured 6% faster (280 vs 297 us on the 4B-like layer at head_dim 256).
inline int pick_mb(int head_dim, int rows_per_req) {
  const int mb = (rows_per_req + 63) / 64;
  const int cap = head_dim == 256 ? 1 : 3;
  return mb < 1 ? 1 : (mb > cap ? cap : mb);
}
// Rows per workgroup the prefix kernel takes at most for this shape (so the host
// can size the grid before launching).
inline int prefix_rows_per_tile(int dtype, int head_dim, int rows_per_req) {
  if (dtype == BSP_F32) return 4;
  return 64 * pick_mb(head_dim, rows_per_req);
}
// Prefill (bsp_prefill_attn): at most this many 16-row query blocks per wave
// (64 * mb query rows per work item); the plan takes fewer when the batch is
// too small to give every CU two workgroups.
constexpr int prefill_max_mb(int head_dim) { return head_dim == 256 ? 2 : 3; }
// Workgroups that fill the chip once: two per CU on the 256 CUs of an MI355X.
constexpr int kFillBlocks = 512;
hipError_t launch_prefill(const PrefixParams& p, const FusedParams& f, int dtype, int head_dim,
                          int mb, int n_items, hipStream_t s);
// A mixed step in one launch (beam-step workgroups beside context workgroups):
// one query block per wave on both sides, head_dim <= 128, the beam step's
// tails in the LDS slot table and no split request.
bool mixed_step_supported(const PrefixParams& dp, const FusedParams& df, int dtype, int head_dim,
                          int rows_per_req, int tail_pad, int pre_mb);
hipError_t launch_mixed_step(const PrefixParams& dp, const FusedParams& df, const PrefixParams& pp,
                             const FusedParams& pf, int dtype, int head_dim, int n_pre_items,
                             hipStream_t s);
hipError_t launch_tail(const TailParams& p, int dtype, int head_dim, hipStream_t s);
hipError_t launch_tail_slots(const TailParams& p, hipStream_t s);
hipError_t launch_merge(const MergeParams& p, int out_dtype, hipStream_t s);
hipError_t launch_naive(const TailParams& p, void* o_out, float* lse_out, int dtype,
                        int head_dim, hipStream_t s);

}  // namespace bsp
