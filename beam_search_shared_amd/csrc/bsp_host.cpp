// Host side of libbsp: the per-step planner, argument validation and the C
// entry points declared in include/bsp.h.
//
// The plan is built once per step on the host and read by every layer of that
// step (TensorRT-LLM PR #21738, "Add opt-in cascade attention for wide beam
// search on KVCM V2", first commit message). It validates lengths and page ids
// and raises rather than clamping a bad prompt page index (eligibility commit),
// rejects a tail longer than a fixed maximum (review thread on MAX_TAIL), takes
// the shared prompt's page table from beam 0 (KV-cache-manager-V2 commit), and
// hands its tables to the device through pinned staging and an asynchronous
// copy, without waiting for the stream (commit making re-planning non-blocking).
// In cached-prefix mode it bounds each request's keys to the valid prefix
// rounded up to the key bucket, capped at the allocation, one row for an empty
// cache (Phi-4 cached-prefix PR, TensorRT-Model-Connect #2202: Exit Criteria,
// Implementation).
#include <algorithm>
#include <array>
#include <functional>
#include <queue>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "bsp_internal.h"
#include "merge_row.h"

using bsp::DevHeader;
using bsp::ReqInfo;

namespace {

thread_local std::string g_last_error;

bsp_status_t fail(bsp_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

bsp_status_t ok() {
  g_last_error.clear();
  return BSP_OK;
}

bsp_status_t hip_fail(hipError_t e, const char* what) {
  return fail(BSP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

int log2i(int32_t x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int elem_bytes(int dtype) { return dtype == BSP_F32 ? 4 : 2; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

// Cost model of the fused step's split (in keys of one KV head streamed by one
// workgroup): the fixed work of a workgroup (its start, and the tails, output
// and token write that end a request), and the partial-state traffic a split
// adds, counted in keys of the same bytes. A split must shorten the modelled
// step by this fraction to be taken.
constexpr int64_t kItemOverheadKeys = 160;
constexpr double kSplitMinGain = 0.05;

struct bsp_plan_s {
  bsp_layer_desc_t desc;
  int32_t max_requests = 0, max_beam = 0, max_blocks = 0, max_seq_len = 0, max_q_len = 0;
  uint32_t flags = 0;
  bool host_only = false;
  bool check_mode = false;
  int page_shift = 0;
  size_t ws_bytes = 0;
  // the fused step's work items and split partial states (beam decode plans)
  int32_t max_fitems = 0, max_qt = 0, max_slots = 0, part_floats = 0;
  int32_t split_force = -1;  // BSP_SPLIT: -1 automatic, 0 never, > 0 chunk of that many keys
  size_t fitems_off = 0, split_count_off = 0, split_part_off = 0;
  // prefill work list (bsp_plan_prefill): (request, query tile) int32 pairs
  int32_t max_items = 0;
  size_t items_off = 0;

  // staging ring (pinned host memory, or malloc for host-only plans)
  void* staging[2] = {nullptr, nullptr};
  hipEvent_t staged[2] = {nullptr, nullptr};
  bool staged_pending[2] = {false, false};
  int ring = 0;

  // current plan
  bool planned = false;
  int32_t B = 0, W = 0, q_len = 0, tail_pad = 0, n_split = 1, rows_per_req = 0;
  int32_t n_fitems = 0, n_slots = 0;  // fused-step items and split partial slots in use
  int32_t split_keys = 0;  // keys per split of the current step (0: one pass)
  int32_t prefix_rpt = 0;  // query rows per work item of bsp_prefix_attn
  void* ws_d = nullptr;
  void* zeroed_ws = nullptr;  // workspace whose header this plan has cleared
  std::vector<ReqInfo> h_req;
  std::vector<bsp::FusedItem> h_fitems;
  std::vector<int32_t> h_pages;
  // prefill plans (bsp_plan_prefill): ragged query rows, work list
  bool prefill = false;
  int32_t rows_total = 0, n_items = 0, prefill_mb = 1;
};

namespace {

size_t req_offset() { return bsp::kHeaderBytes; }
// header | ReqInfo[B] | page table | (fixed offsets, sized for the plan's
// capacity) fused-step items | split counters | split partial states |
// prefill work list
size_t pages_offset(int32_t B) { return align_up(bsp::kHeaderBytes + sizeof(ReqInfo) * B, 16); }

DevHeader* dev_header(const bsp_plan_s* pl) { return static_cast<DevHeader*>(pl->ws_d); }
const ReqInfo* dev_req(const bsp_plan_s* pl) {
  return reinterpret_cast<const ReqInfo*>(static_cast<char*>(pl->ws_d) + req_offset());
}
const int32_t* dev_pages(const bsp_plan_s* pl) {
  return reinterpret_cast<const int32_t*>(static_cast<char*>(pl->ws_d) + pages_offset(pl->B));
}

int32_t bucket_rows(int32_t valid, int32_t bucket, int32_t cap) {
  if (valid <= 0) return 1;
  const int64_t r = ceil_div(valid, bucket) * bucket;
  return (int32_t)(r < cap ? r : cap);
}

bsp_status_t check_device_ready(const bsp_plan_s* pl) {
  if (pl == nullptr) return fail(BSP_ERR_ARG, "null plan");
  if (!pl->planned)
    return fail(BSP_ERR_STALE_PLAN, "plan has no valid step: call bsp_plan first");
  if (pl->host_only) return fail(BSP_ERR_ARG, "host-only plan cannot launch kernels");
  return BSP_OK;
}

// Entry points of the beam step need a bsp_plan step; bsp_prefill_attn needs a
// bsp_plan_prefill step.
bsp_status_t check_beam_ready(const bsp_plan_s* pl) {
  const bsp_status_t st = check_device_ready(pl);
  if (st != BSP_OK) return st;
  if (pl->prefill) return fail(BSP_ERR_ARG, "plan holds a prefill step (bsp_plan_prefill)");
  return BSP_OK;
}

// Check mode: wait for the launch and surface any recorded index fault.
bsp_status_t after_launch(bsp_plan_s* pl, hipError_t launch, const char* what,
                          hipStream_t stream) {
  if (launch != hipSuccess) return hip_fail(launch, what);
  if (pl != nullptr && pl->check_mode) return bsp_check(pl, stream);
  return ok();
}

}  // namespace

namespace bsp {

bsp_status_t set_error(bsp_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

void forget_workspace(bsp_plan_t plan) {
  if (plan != nullptr) plan->zeroed_ws = nullptr;
}

}  // namespace bsp

extern "C" {

const char* bsp_last_error(void) { return g_last_error.c_str(); }

int32_t bsp_version(void) { return 100; }

bsp_status_t bsp_plan_create(const bsp_layer_desc_t* desc, int32_t max_requests,
                             int32_t max_beam, int32_t max_blocks_per_seq, int32_t max_seq_len,
                             int32_t max_q_len, uint32_t flags, bsp_plan_t* out) {
  if (out == nullptr || desc == nullptr) return fail(BSP_ERR_ARG, "null argument");
  *out = nullptr;
  const bsp_layer_desc_t& d = *desc;
  if (d.dtype != BSP_F32 && d.dtype != BSP_F16 && d.dtype != BSP_BF16)
    return fail(BSP_ERR_DTYPE, "dtype %d is not one of f32, f16, bf16", d.dtype);
  if (d.num_q_heads <= 0 || d.num_kv_heads <= 0 || d.num_q_heads % d.num_kv_heads != 0)
    return fail(BSP_ERR_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                d.num_q_heads, d.num_kv_heads);
  if (d.head_dim != 64 && d.head_dim != 128 && d.head_dim != 256)
    return fail(BSP_ERR_UNSUPPORTED, "head_dim %d is not 64, 128 or 256", d.head_dim);
  if (!is_pow2(d.page_size) || d.page_size > 1024)
    return fail(BSP_ERR_UNSUPPORTED, "page_size %d is not a power of two <= 1024", d.page_size);
  if (d.num_pages <= 0) return fail(BSP_ERR_ARG, "num_pages must be positive");
  if ((int64_t)d.num_pages * d.page_size > INT32_MAX)
    return fail(BSP_ERR_UNSUPPORTED, "num_pages * page_size exceeds the int32 slot range");
  if (!(d.sm_scale >= 0.f) || std::isinf(d.sm_scale))
    return fail(BSP_ERR_ARG, "sm_scale must be finite and >= 0");
  if (d.max_tail < 0) return fail(BSP_ERR_ARG, "max_tail must be >= 0");
  if (d.key_bucket < 0) return fail(BSP_ERR_ARG, "key_bucket must be >= 0");
  if (d.key_bucket > 0 && d.max_cache_rows <= 0)
    return fail(BSP_ERR_ARG, "cached-prefix mode needs max_cache_rows > 0");
  if (d.mask != BSP_MASK_NONE && d.mask != BSP_MASK_CAUSAL)
    return fail(BSP_ERR_ARG, "mask %d is not NONE or CAUSAL", d.mask);
  if (d.kv_split < -1 || (d.kv_split > 0 && d.kv_split % 64 != 0))
    return fail(BSP_ERR_ARG, "kv_split (%d) must be -1, 0 or a positive multiple of 64",
                d.kv_split);
  if (max_requests <= 0 || max_beam <= 0 || max_blocks_per_seq <= 0 || max_seq_len <= 0 ||
      max_q_len <= 0)
    return fail(BSP_ERR_ARG, "capacities must be positive");
  if ((int64_t)max_blocks_per_seq * d.page_size < max_seq_len)
    return fail(BSP_ERR_ARG, "max_blocks_per_seq * page_size (%lld) < max_seq_len (%d)",
                (long long)max_blocks_per_seq * d.page_size, max_seq_len);
  if (d.key_bucket > 0 && (int64_t)max_blocks_per_seq * d.page_size < d.max_cache_rows)
    return fail(BSP_ERR_ARG, "block tables cannot cover max_cache_rows");

  bsp_plan_s* pl = new bsp_plan_s();
  pl->desc = d;
  if (pl->desc.sm_scale == 0.f) pl->desc.sm_scale = 1.0f / std::sqrt((float)d.head_dim);
  pl->max_requests = max_requests;
  pl->max_beam = max_beam;
  pl->max_blocks = max_blocks_per_seq;
  pl->max_seq_len = max_seq_len;
  pl->max_q_len = max_q_len;
  pl->flags = flags;
  pl->host_only = (flags & BSP_PLAN_HOST_ONLY) != 0;
  const char* env = std::getenv("BSP_CHECK");
  pl->check_mode = env != nullptr && env[0] == '1';
  pl->page_shift = log2i(d.page_size);
  pl->ws_bytes = align_up(pages_offset(max_requests) +
                              sizeof(int32_t) * (size_t)max_requests * max_blocks_per_seq,
                          256);
  // The fused step's items (one per request, or one per chunk of a split
  // prompt), then, when the geometry allows a split, an arrival counter per
  // (request, KV head, query tile) and the partial states of split chunks,
  // at most kSplitPartBudget bytes of them and 16 chunks per request on
  // average.
  {
    const int G = d.num_q_heads / d.num_kv_heads;
    const int64_t rows = (int64_t)max_beam * G;
    // query blocks per wave and query tiles grow with the rows per request
    const int mb = bsp::pick_mb(d.head_dim, (int)std::min<int64_t>(rows, INT32_MAX / 2));
    pl->max_qt = (int32_t)ceil_div(rows, 64 * mb);
    pl->part_floats = bsp::split_part_floats(d.head_dim, mb);
    const size_t slot_bytes =
        sizeof(float) * 256 * (size_t)pl->part_floats * d.num_kv_heads * pl->max_qt;
    const bool capable = d.key_bucket == 0 && d.dtype != BSP_F32;
    pl->max_slots = capable ? (int32_t)std::min<size_t>((size_t)16 * max_requests,
                                                       bsp::kSplitPartBudget / slot_bytes)
                            : 0;
    if (pl->max_slots < 2) pl->max_slots = 0;
    const char* env = std::getenv("BSP_SPLIT");
    pl->split_force = env == nullptr || env[0] == '\0' ? -1 : std::atoi(env);
    if (pl->split_force > 0) pl->split_force = (int32_t)(ceil_div(pl->split_force, 64) * 64);
    pl->max_fitems = max_requests + pl->max_slots;
    pl->fitems_off = pl->ws_bytes;
    pl->split_count_off =
        align_up(pl->fitems_off + sizeof(bsp::FusedItem) * (size_t)pl->max_fitems, 256);
    pl->split_part_off = align_up(pl->split_count_off + sizeof(int32_t) * (size_t)max_requests *
                                                            d.num_kv_heads * pl->max_qt,
                                  256);
    pl->ws_bytes = align_up(pl->split_part_off + slot_bytes * (size_t)pl->max_slots, 256);
  }
  // Prefill work list: at most one item per 64 query rows of each request.
  {
    const int G = d.num_q_heads / d.num_kv_heads;
    pl->max_items = (int32_t)std::min<int64_t>(
        INT32_MAX / 2, (int64_t)max_requests * ceil_div((int64_t)max_q_len * G, 64));
    pl->items_off = pl->ws_bytes;
    pl->ws_bytes = align_up(pl->items_off + 2 * sizeof(int32_t) * (size_t)pl->max_items, 256);
  }
  for (int i = 0; i < 2; ++i) {
    if (pl->host_only) {
      pl->staging[i] = std::calloc(1, pl->ws_bytes);
      if (pl->staging[i] == nullptr) {
        bsp_plan_destroy(pl);
        return fail(BSP_ERR_ARG, "out of host memory");
      }
      continue;
    }
    hipError_t e = hipHostMalloc(&pl->staging[i], pl->ws_bytes, hipHostMallocDefault);
    if (e != hipSuccess) {
      pl->staging[i] = nullptr;
      bsp_plan_destroy(pl);
      return hip_fail(e, "hipHostMalloc (plan staging)");
    }
    std::memset(pl->staging[i], 0, pl->ws_bytes);
    e = hipEventCreateWithFlags(&pl->staged[i], hipEventDisableTiming);
    if (e != hipSuccess) {
      pl->staged[i] = nullptr;
      bsp_plan_destroy(pl);
      return hip_fail(e, "hipEventCreate (plan staging)");
    }
  }
  *out = pl;
  return ok();
}

size_t bsp_plan_workspace_bytes(bsp_plan_t plan) { return plan ? plan->ws_bytes : 0; }

void bsp_plan_destroy(bsp_plan_t plan) {
  if (plan == nullptr) return;
  for (int i = 0; i < 2; ++i) {
    if (plan->staged[i] != nullptr) {
      if (plan->staged_pending[i]) (void)hipEventSynchronize(plan->staged[i]);
      (void)hipEventDestroy(plan->staged[i]);
    }
    if (plan->staging[i] != nullptr) {
      if (plan->host_only) std::free(plan->staging[i]);
      else (void)hipHostFree(plan->staging[i]);
    }
  }
  delete plan;
}

bsp_status_t bsp_plan(bsp_plan_t pl, int32_t B, int32_t W, int32_t q_len,
                      const int32_t* prefix_len_h, const int32_t* seq_len_h,
                      const int32_t* block_tables_h, void* workspace_d, size_t workspace_bytes,
                      hipStream_t stream) {
  if (pl == nullptr) return fail(BSP_ERR_ARG, "null plan");
  pl->planned = false;
  if (B < 1 || B > pl->max_requests)
    return fail(BSP_ERR_ARG, "B = %d outside [1, %d]", B, pl->max_requests);
  if (W < 1 || W > pl->max_beam) return fail(BSP_ERR_ARG, "W = %d outside [1, %d]", W, pl->max_beam);
  if (q_len < 1 || q_len > pl->max_q_len)
    return fail(BSP_ERR_ARG, "q_len = %d outside [1, %d]", q_len, pl->max_q_len);
  if (prefix_len_h == nullptr || seq_len_h == nullptr || block_tables_h == nullptr)
    return fail(BSP_ERR_ARG, "null host table");
  if (pl->host_only) {
    if (workspace_d != nullptr) return fail(BSP_ERR_ARG, "host-only plan takes no workspace");
  } else {
    if (workspace_d == nullptr) return fail(BSP_ERR_WORKSPACE, "null workspace");
    if (workspace_bytes < pl->ws_bytes)
      return fail(BSP_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes,
                  pl->ws_bytes);
    if ((reinterpret_cast<uintptr_t>(workspace_d) & 255u) != 0)
      return fail(BSP_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }

  const bsp_layer_desc_t& d = pl->desc;
  const int ps = d.page_size;
  const int MB = pl->max_blocks;
  const bool cached = d.key_bucket > 0;
  auto bt = [&](int b, int k, int i) -> int32_t {
    return block_tables_h[((int64_t)b * W + k) * MB + i];
  };

  std::vector<ReqInfo> req(B);
  int64_t total_pages = 0;
  int32_t max_tail_seen = 0, n_split = 1;
  for (int b = 0; b < B; ++b) {
    const int32_t P = prefix_len_h[b], S = seq_len_h[b];
    ReqInfo& r = req[b];
    std::memset(&r, 0, sizeof(r));
    if (cached) {
      if (P < 0 || P > d.max_cache_rows)
        return fail(BSP_ERR_ARG, "request %d: valid rows %d outside [0, %d]", b, P,
                    d.max_cache_rows);
      if (S != P)
        return fail(BSP_ERR_ARG, "request %d: cached-prefix mode needs seq_len == prefix_len", b);
      r.n_keys = bucket_rows(P, d.key_bucket, d.max_cache_rows);
      r.valid = P;
    } else {
      if (P < 0 || S < P || S > pl->max_seq_len)
        return fail(BSP_ERR_ARG, "request %d: need 0 <= prefix_len (%d) <= seq_len (%d) <= %d", b,
                    P, S, pl->max_seq_len);
      const int32_t T = S - P;
      if (d.max_tail > 0 && T > d.max_tail)
        return fail(BSP_ERR_TAIL_OVERFLOW,
                    "request %d: a beam carries %d tail positions but the plan's fixed tail "
                    "length is %d",
                    b, T, d.max_tail);
      r.n_keys = P;
      r.valid = P;
      r.tail = T;
      if (T > max_tail_seen) max_tail_seen = T;
    }
    r.prefix = P;
    r.seq = S;
    const int64_t nblk = ceil_div(r.n_keys, ps);
    if (nblk > MB) return fail(BSP_ERR_ARG, "request %d: %lld blocks > max_blocks %d", b,
                               (long long)nblk, MB);
    for (int64_t i = 0; i < nblk; ++i) {
      const int32_t pg = bt(b, 0, (int)i);
      if (pg < 0 || pg >= d.num_pages)
        return fail(BSP_ERR_PAGE_INDEX, "request %d beam 0 block %lld: page id %d outside [0, %d)",
                    b, (long long)i, pg, d.num_pages);
    }
    if (!cached && S > P) {  // every beam's tail blocks may be read through the indirection
      for (int k = 0; k < W; ++k)
        for (int i = P / ps; i <= (S - 1) / ps; ++i) {
          const int32_t pg = bt(b, k, i);
          if (pg < 0 || pg >= d.num_pages)
            return fail(BSP_ERR_PAGE_INDEX, "request %d beam %d block %d: page id %d outside [0, %d)",
                        b, k, i, pg, d.num_pages);
        }
    }
    if (pl->check_mode && !cached) {
      for (int k = 1; k < W; ++k)
        for (int i = 0; i < P / ps; ++i)
          if (bt(b, k, i) != bt(b, 0, i))
            return fail(BSP_ERR_ARG,
                        "check mode: request %d beam %d does not share prompt block %d with beam 0",
                        b, k, i);
    }
    r.page_off = (int32_t)total_pages;
    total_pages += nblk;
  }

  // Key split: fixed, none, or (kv_split = -1) the smallest multiple of 64
  // keys whose work items (request, KV head, split, query tile) still fit one
  // round of two workgroups per CU; a split above the longest key range is no
  // split.
  int32_t split_keys = d.kv_split > 0 ? d.kv_split : 0;
  if (d.kv_split < 0) {
    const int rows = W * q_len * (d.num_q_heads / d.num_kv_heads);
    const int64_t n_qt = ceil_div(rows, bsp::prefix_rows_per_tile(d.dtype, d.head_dim, rows));
    int32_t v_max = 0;
    for (int b = 0; b < B; ++b) v_max = std::max(v_max, req[b].valid);
    auto items = [&](int64_t s) {
      int64_t n = 0;
      for (int b = 0; b < B; ++b) n += std::max<int64_t>(1, ceil_div(req[b].valid, s));
      return n * d.num_kv_heads * n_qt;
    };
    int64_t s = 64;
    while (s < v_max && items(s) > bsp::kFillBlocks) s += 64;
    split_keys = s < v_max ? (int32_t)s : 0;
  }
  for (int b = 0; b < B; ++b) {
    ReqInfo& r = req[b];
    r.n_split = split_keys > 0 ? (int32_t)(r.valid > 0 ? ceil_div(r.valid, split_keys) : 1) : 1;
    if (r.n_split > n_split) n_split = r.n_split;
  }
  // Query rows per work item of bsp_prefix_attn: the tallest tile whose grid
  // still gives every CU two workgroups (without a key split), else one 16-row
  // block per wave. A one-request causal segment of 2000 rows then runs as 752
  // items of 64 rows instead of 256 items of 192, one per CU.
  const int rows_req = W * q_len * (d.num_q_heads / d.num_kv_heads);
  int32_t prefix_rpt = bsp::prefix_rows_per_tile(d.dtype, d.head_dim, rows_req);
  if (d.dtype != BSP_F32 && split_keys == 0) {
    for (; prefix_rpt > 64; prefix_rpt -= 64)
      if ((int64_t)B * d.num_kv_heads * ceil_div(rows_req, prefix_rpt) >= bsp::kFillBlocks) break;
  }

  // Fill the staging buffer: header (zero), request info, page table.
  const int slot = pl->ring;
  if (pl->staged_pending[slot]) {
    const hipError_t e = hipEventSynchronize(pl->staged[slot]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize (plan staging)");
    pl->staged_pending[slot] = false;
  }
  char* st = static_cast<char*>(pl->staging[slot]);
  std::memset(st, 0, bsp::kHeaderBytes);
  std::memcpy(st + req_offset(), req.data(), sizeof(ReqInfo) * B);
  int32_t* pg_out = reinterpret_cast<int32_t*>(st + pages_offset(B));
  std::vector<int32_t> pages((size_t)total_pages);
  for (int b = 0; b < B; ++b)
    for (int64_t i = 0; i < ceil_div(req[b].n_keys, ps); ++i)
      pages[(size_t)req[b].page_off + i] = bt(b, 0, (int)i);
  if (!pages.empty()) std::memcpy(pg_out, pages.data(), sizeof(int32_t) * pages.size());

  // The fused step's work items (beam decode, bf16/f16): one per request, or
  // one per chunk of a request whose prompt the plan splits. Blocks are
  // dispatched in order and a slot that frees up takes the next block, so the
  // items are listed longest first (the longest-processing-time rule). A split
  // is taken when it shortens the modelled step (items dealt longest first to
  // the slots of one round of workgroups, each item costing its keys, a fixed
  // per-workgroup amount and the partial-state traffic of a split) by
  // kSplitMinGain, or always with BSP_SPLIT=<keys>, never with BSP_SPLIT=0.
  std::vector<bsp::FusedItem> fitems;
  int32_t n_slots = 0, fused_qt = 1;
  const bool fused_ok = q_len == 1 && !cached && d.dtype != BSP_F32;
  if (fused_ok) {
    const int rows_g = W * (d.num_q_heads / d.num_kv_heads);
    fused_qt = (int32_t)ceil_div(rows_g, bsp::prefix_rows_per_tile(d.dtype, d.head_dim, rows_g));
    const int64_t slots =
        std::max<int64_t>(1, bsp::kFillBlocks / ((int64_t)d.num_kv_heads * fused_qt));
    const int mb = bsp::pick_mb(d.head_dim, rows_g);
    const int64_t key_bytes = 2 * (int64_t)d.head_dim * elem_bytes(d.dtype);
    const int64_t part_keys =
        (int64_t)bsp::split_part_floats(d.head_dim, mb) * 256 * 4 / key_bytes;
    std::vector<int32_t> by_len(B);
    for (int b = 0; b < B; ++b) by_len[b] = b;
    std::stable_sort(by_len.begin(), by_len.end(),
                     [&](int32_t x, int32_t y) { return req[x].valid > req[y].valid; });
    // chunks of each request under a candidate chunk size (0: whole): the
    // requests are taken longest first, and each one is split if its chunks
    // still fit the plan's partial-state slots that are left
    auto chunking = [&](int64_t ck, std::vector<int32_t>& parts_of) {
      parts_of.assign(B, 1);
      int64_t used = 0;
      for (int32_t b : by_len) {
        const int64_t n = ck > 0 && req[b].valid > ck ? ceil_div(req[b].valid, ck) : 1;
        if (n > 1 && used + n <= pl->max_slots &&
            (int64_t)B + used + n <= pl->max_fitems) {
          parts_of[b] = (int32_t)n;
          used += n;
        }
      }
    };
    auto model = [&](int64_t ck, const std::vector<int32_t>& parts_of) {
      std::vector<int64_t> cost;
      for (int b = 0; b < B; ++b) {
        const int64_t P = req[b].valid;
        if (parts_of[b] == 1) {
          cost.push_back(P + kItemOverheadKeys);
          continue;
        }
        for (int j = 0; j < parts_of[b]; ++j) {
          const int64_t len = std::min<int64_t>(P, (j + 1) * ck) - j * ck;
          cost.push_back(len + kItemOverheadKeys + part_keys +
                         (j == 0 ? (parts_of[b] - 1) * part_keys : 0));
        }
      }
      std::sort(cost.begin(), cost.end(), std::greater<int64_t>());
      std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> load;
      for (int64_t i = 0; i < std::min<int64_t>(slots, (int64_t)cost.size()); ++i) load.push(0);
      int64_t span = 0;
      for (int64_t c : cost) {
        const int64_t t = load.top() + c;
        load.pop();
        load.push(t);
        span = std::max(span, t);
      }
      return span;
    };
    int64_t ck = 0;
    std::vector<int32_t> parts_of(B, 1);
    if (pl->split_force > 0) {
      ck = pl->split_force;
      chunking(ck, parts_of);
    } else if (pl->split_force < 0 && pl->max_slots > 0 && B > 0) {
      const int64_t p_max = req[by_len[0]].valid;
      const int64_t base = model(0, parts_of);
      int64_t best = base;
      std::vector<int32_t> cand;
      for (int n = 2; n <= 4; ++n) {
        const int64_t c = ceil_div(ceil_div(p_max, n), 64) * 64;
        if (c <= 0 || c >= p_max) continue;
        chunking(c, cand);
        const int64_t span = model(c, cand);
        if (span < best && span <= (int64_t)((1.0 - kSplitMinGain) * base)) {
          best = span;
          ck = c;
          parts_of = cand;
        }
      }
    }
    for (int b = 0; b < B; ++b) {
      const int32_t n = parts_of[b];
      for (int32_t j = 0; j < n; ++j) {
        bsp::FusedItem it;
        std::memset(&it, 0, sizeof(it));
        it.ri = req[b];
        it.b = b;
        it.k_lo = n > 1 ? (int32_t)(j * ck) : 0;
        it.k_hi = n > 1 ? (int32_t)std::min<int64_t>(req[b].valid, (j + 1) * ck) : req[b].valid;
        it.part = j;
        it.parts = n;
        it.slot = n > 1 ? n_slots : -1;
        fitems.push_back(it);
      }
      if (n > 1) n_slots += n;
    }
    // Dealt longest first. When the items fill more than one round of
    // workgroups, a request's tail rows count too (W rows per tail position,
    // each the bytes of one prompt key, carried by its last chunk), so that
    // the items a slot runs one after the other even out; within one round
    // every item starts at once and the order only places them, and the prompt
    // keys alone decide (measured: the wide-beam step 1-1.5% shorter with the
    // tails counted, the 0.6B shape's single round 1.7% longer).
    const bool several_rounds = (int64_t)fitems.size() > slots;
    auto deal_cost = [&](const bsp::FusedItem& x) {
      int64_t c = x.k_hi - x.k_lo;
      if (several_rounds && x.k_hi == x.ri.valid) c += (int64_t)W * x.ri.tail;
      return c;
    };
    std::stable_sort(fitems.begin(), fitems.end(),
                     [&](const bsp::FusedItem& x, const bsp::FusedItem& y) {
                       return deal_cost(x) > deal_cost(y);
                     });
    // In one round the order only places items. Workgroup i goes to XCD i % 8,
    // so with 8 KV heads every XCD gets one head of each item, in list order;
    // listing the shorter half shortest first puts the k-th longest and the
    // k-th shortest item k and k + n/2 places apart, side by side on a CU if
    // each XCD's CUs take its workgroups in turn (measured in two runs: head_dim
    // 64 2%, n-sample 0.7-0.9%, the 4B-like layer 0-0.9%, the 0.6B shape 0-1.4%
    // shorter, head_dim 256 unchanged; interleaving longest and shortest item by
    // item was slower).
    if (!several_rounds) std::reverse(fitems.begin() + fitems.size() / 2, fitems.end());
    std::memcpy(st + pl->fitems_off, fitems.data(), sizeof(bsp::FusedItem) * fitems.size());
    if (n_slots > 0)
      std::memset(st + pl->split_count_off, 0,
                  sizeof(int32_t) * (size_t)B * d.num_kv_heads * fused_qt);
  }

  // One-row cached-prefix decode (bsp_cached_decode): an arrival counter per
  // (request, KV head), zero at every launch (the last chunk resets it).
  const bool cached_decode = cached && q_len == 1 && W == 1;
  if (cached_decode)
    std::memset(st + pl->split_count_off, 0, sizeof(int32_t) * (size_t)B * d.num_kv_heads);

  if (!pl->host_only) {
    size_t end = pages_offset(B) + sizeof(int32_t) * pages.size();
    if (!fitems.empty()) end = pl->fitems_off + sizeof(bsp::FusedItem) * fitems.size();
    if (n_slots > 0)
      end = pl->split_count_off + sizeof(int32_t) * (size_t)B * d.num_kv_heads * fused_qt;
    if (cached_decode) end = pl->split_count_off + sizeof(int32_t) * (size_t)B * d.num_kv_heads;
    const size_t begin = workspace_d == pl->zeroed_ws ? req_offset() : 0;
    hipError_t e = hipMemcpyAsync(static_cast<char*>(workspace_d) + begin, st + begin,
                                  end - begin, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (plan tables)");
    e = hipEventRecord(pl->staged[slot], stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord (plan staging)");
    pl->staged_pending[slot] = true;
    pl->ring = 1 - slot;
    pl->zeroed_ws = workspace_d;
  }

  pl->B = B;
  pl->W = W;
  pl->q_len = q_len;
  pl->tail_pad = d.max_tail > 0 ? d.max_tail : max_tail_seen;
  pl->n_split = n_split;
  pl->split_keys = split_keys;
  pl->prefix_rpt = prefix_rpt;
  pl->rows_per_req = W * q_len * (d.num_q_heads / d.num_kv_heads);
  pl->n_fitems = (int32_t)fitems.size();
  pl->n_slots = n_slots;
  pl->h_fitems = std::move(fitems);
  pl->prefill = false;
  pl->rows_total = B * W * q_len;
  pl->n_items = 0;
  pl->ws_d = workspace_d;
  pl->h_req = std::move(req);
  pl->h_pages = std::move(pages);
  pl->planned = true;
  return ok();
}

int32_t bsp_plan_num_splits(bsp_plan_t pl) { return pl && pl->planned ? pl->n_split : -1; }
int32_t bsp_plan_split_keys(bsp_plan_t pl) { return pl && pl->planned ? pl->split_keys : -1; }
int32_t bsp_plan_tail_len(bsp_plan_t pl) { return pl && pl->planned ? pl->tail_pad : -1; }

bsp_status_t bsp_plan_prefill(bsp_plan_t pl, int32_t C, const int32_t* q_len_h,
                              const int32_t* cached_len_h, const int32_t* block_tables_h,
                              void* workspace_d, size_t workspace_bytes, hipStream_t stream) {
  if (pl == nullptr) return fail(BSP_ERR_ARG, "null plan");
  pl->planned = false;
  const bsp_layer_desc_t& d = pl->desc;
  if (d.key_bucket > 0) return fail(BSP_ERR_ARG, "prefill steps need a plan without key_bucket");
  if (C < 1 || C > pl->max_requests)
    return fail(BSP_ERR_ARG, "C = %d outside [1, %d]", C, pl->max_requests);
  if (q_len_h == nullptr || cached_len_h == nullptr || block_tables_h == nullptr)
    return fail(BSP_ERR_ARG, "null host table");
  if (pl->host_only) {
    if (workspace_d != nullptr) return fail(BSP_ERR_ARG, "host-only plan takes no workspace");
  } else {
    if (workspace_d == nullptr) return fail(BSP_ERR_WORKSPACE, "null workspace");
    if (workspace_bytes < pl->ws_bytes)
      return fail(BSP_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes,
                  pl->ws_bytes);
    if ((reinterpret_cast<uintptr_t>(workspace_d) & 255u) != 0)
      return fail(BSP_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  const int ps = d.page_size;
  const int MBLK = pl->max_blocks;
  const int G = d.num_q_heads / d.num_kv_heads;
  // Query rows per work item: the tallest tile (most reuse of each key tile)
  // that still gives every CU two workgroups, else the shortest.
  int mb = bsp::prefill_max_mb(d.head_dim);
  for (; mb > 1; --mb) {
    int64_t n = 0;
    for (int b = 0; b < C; ++b) n += ceil_div((int64_t)std::max(q_len_h[b], 0) * G, 64 * mb);
    if (n * d.num_kv_heads >= bsp::kFillBlocks) break;
  }
  const int rpt = 64 * mb;
  std::vector<ReqInfo> req(C);
  std::vector<int32_t> pages;
  std::vector<std::array<int32_t, 3>> items;  // (keys, request, tile)
  int64_t rows = 0;
  for (int b = 0; b < C; ++b) {
    const int32_t Sq = q_len_h[b], L = cached_len_h[b];
    if (Sq < 1 || Sq > pl->max_q_len)
      return fail(BSP_ERR_ARG, "request %d: chunk of %d rows outside [1, %d]", b, Sq,
                  pl->max_q_len);
    if (L < 0 || (int64_t)L + Sq > pl->max_seq_len)
      return fail(BSP_ERR_ARG, "request %d: need 0 <= cached (%d) and cached + chunk (%lld) <= %d",
                  b, L, (long long)L + Sq, pl->max_seq_len);
    ReqInfo& r = req[b];
    std::memset(&r, 0, sizeof(r));
    r.n_keys = r.valid = r.seq = L + Sq;
    r.prefix = L;
    r.tail = Sq;
    r.n_split = 1;
    r.q_off = (int32_t)rows;
    r.page_off = (int32_t)pages.size();
    const int64_t nblk = ceil_div(r.n_keys, ps);
    if (nblk > MBLK)
      return fail(BSP_ERR_ARG, "request %d: %lld blocks > max_blocks %d", b, (long long)nblk, MBLK);
    for (int64_t i = 0; i < nblk; ++i) {
      const int32_t pg = block_tables_h[(int64_t)b * MBLK + i];
      if (pg < 0 || pg >= d.num_pages)
        return fail(BSP_ERR_PAGE_INDEX, "request %d block %lld: page id %d outside [0, %d)", b,
                    (long long)i, pg, d.num_pages);
      pages.push_back(pg);
    }
    const int32_t nqt = (int32_t)ceil_div((int64_t)Sq * G, rpt);
    for (int32_t qt = 0; qt < nqt; ++qt) {
      const int64_t last = std::min<int64_t>((int64_t)(qt + 1) * rpt, (int64_t)Sq * G) - 1;
      items.push_back({(int32_t)(L + last / G + 1), b, qt});
    }
    rows += Sq;
  }
  if (rows > INT32_MAX / 2) return fail(BSP_ERR_ARG, "too many query rows (%lld)", (long long)rows);
  if ((int64_t)items.size() > pl->max_items)
    return fail(BSP_ERR_ARG, "%zu work items > %d", items.size(), pl->max_items);
  // Longest key range first: the items that stream the most keys start in the
  // first round of workgroups, the short ones fill in behind them.
  std::stable_sort(items.begin(), items.end(),
                   [](const std::array<int32_t, 3>& x, const std::array<int32_t, 3>& y) {
                     return x[0] > y[0];
                   });

  const int slot = pl->ring;
  if (pl->staged_pending[slot]) {
    const hipError_t e = hipEventSynchronize(pl->staged[slot]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize (plan staging)");
    pl->staged_pending[slot] = false;
  }
  char* st = static_cast<char*>(pl->staging[slot]);
  std::memset(st, 0, bsp::kHeaderBytes);
  std::memcpy(st + req_offset(), req.data(), sizeof(ReqInfo) * C);
  if (!pages.empty())
    std::memcpy(st + pages_offset(C), pages.data(), sizeof(int32_t) * pages.size());
  int32_t* it = reinterpret_cast<int32_t*>(st + pl->items_off);
  for (size_t i = 0; i < items.size(); ++i) {
    it[2 * i] = items[i][1];
    it[2 * i + 1] = items[i][2];
  }
  if (!pl->host_only) {
    const size_t begin = workspace_d == pl->zeroed_ws ? req_offset() : 0;
    const size_t end = pl->items_off + 2 * sizeof(int32_t) * items.size();
    hipError_t e = hipMemcpyAsync(static_cast<char*>(workspace_d) + begin, st + begin,
                                  end - begin, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (prefill tables)");
    e = hipEventRecord(pl->staged[slot], stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord (plan staging)");
    pl->staged_pending[slot] = true;
    pl->ring = 1 - slot;
    pl->zeroed_ws = workspace_d;
  }
  pl->B = C;
  pl->W = 1;
  pl->q_len = 0;
  pl->tail_pad = 0;
  pl->n_split = 1;
  pl->rows_per_req = 0;
  pl->n_fitems = 0;
  pl->n_slots = 0;
  pl->h_fitems.clear();
  pl->prefill = true;
  pl->rows_total = (int32_t)rows;
  pl->n_items = (int32_t)items.size();
  pl->prefill_mb = mb;
  pl->ws_d = workspace_d;
  pl->h_req = std::move(req);
  pl->h_pages = std::move(pages);
  pl->planned = true;
  return ok();
}


namespace {

// Validation and kernel parameters of the current-token write, from the layer
// geometry alone; faults go to `fault` (int32[3]) or nowhere.
bsp_status_t write_kv_params(const bsp_layer_desc_t& d, const void* k_new, const void* v_new,
                             int64_t src_row_stride, const int32_t* slots_d, int32_t n,
                             void* k_pool, void* v_pool, int32_t* fault, bsp::WriteKvParams& p) {
  if (!k_new || !v_new || !slots_d || !k_pool || !v_pool) return fail(BSP_ERR_ARG, "null pointer");
  const int vec = 16 / elem_bytes(d.dtype);
  if (src_row_stride < (int64_t)d.num_kv_heads * d.head_dim || src_row_stride % vec != 0)
    return fail(BSP_ERR_ARG, "src_row_stride %lld must be >= %d and a multiple of %d",
                (long long)src_row_stride, d.num_kv_heads * d.head_dim, vec);
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(BSP_ERR_ARG, "k_new, v_new and the pools must be 16-byte aligned");
  p.k_new = k_new;
  p.v_new = v_new;
  p.src_stride = src_row_stride;
  p.slots = slots_d;
  p.n = n;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.hkv = d.num_kv_heads;
  p.d = d.head_dim;
  p.page_size = d.page_size;
  p.num_slots = (int64_t)d.num_pages * d.page_size;
  p.fault = fault;
  return BSP_OK;
}

}  // namespace

bsp_status_t bsp_write_kv(bsp_plan_t pl, const void* k_new, const void* v_new,
                          int64_t src_row_stride, const int32_t* slots_d, int32_t n, void* k_pool,
                          void* v_pool, hipStream_t stream) {
  bsp_status_t st = check_device_ready(pl);
  if (st != BSP_OK) return st;
  if (n < 0) return fail(BSP_ERR_ARG, "n < 0");
  if (n == 0) return ok();
  bsp::WriteKvParams p;
  st = write_kv_params(pl->desc, k_new, v_new, src_row_stride, slots_d, n, k_pool, v_pool,
                       &dev_header(pl)->error_bits, p);
  if (st != BSP_OK) return st;
  return after_launch(pl, bsp::launch_write_kv(p, pl->desc.dtype, stream), "write_kv launch", stream);
}

bsp_status_t bsp_write_kv_desc(const bsp_layer_desc_t* desc, const void* k_new, const void* v_new,
                               int64_t src_row_stride, const int32_t* slots_d, int32_t n,
                               void* k_pool, void* v_pool, int32_t* faults_d, hipStream_t stream) {
  if (desc == nullptr) return fail(BSP_ERR_ARG, "null descriptor");
  const bsp_layer_desc_t& d = *desc;
  if (d.dtype != BSP_F32 && d.dtype != BSP_F16 && d.dtype != BSP_BF16)
    return fail(BSP_ERR_DTYPE, "dtype %d is not one of f32, f16, bf16", d.dtype);
  if (d.num_kv_heads <= 0) return fail(BSP_ERR_ARG, "num_kv_heads must be positive");
  if (d.head_dim != 64 && d.head_dim != 128 && d.head_dim != 256)
    return fail(BSP_ERR_UNSUPPORTED, "head_dim %d is not 64, 128 or 256", d.head_dim);
  if (!is_pow2(d.page_size) || d.page_size > 1024)
    return fail(BSP_ERR_UNSUPPORTED, "page_size %d is not a power of two <= 1024", d.page_size);
  if (d.num_pages <= 0) return fail(BSP_ERR_ARG, "num_pages must be positive");
  if ((int64_t)d.num_pages * d.page_size > INT32_MAX)
    return fail(BSP_ERR_UNSUPPORTED, "num_pages * page_size exceeds the int32 slot range");
  if (n < 0) return fail(BSP_ERR_ARG, "n < 0");
  if (n == 0) return ok();
  if (faults_d != nullptr && (reinterpret_cast<uintptr_t>(faults_d) & 3u) != 0)
    return fail(BSP_ERR_ARG, "faults_d must be 4-byte aligned");
  bsp::WriteKvParams p;
  const bsp_status_t st =
      write_kv_params(d, k_new, v_new, src_row_stride, slots_d, n, k_pool, v_pool, faults_d, p);
  if (st != BSP_OK) return st;
  const hipError_t e = bsp::launch_write_kv(p, d.dtype, stream);
  if (e != hipSuccess) return hip_fail(e, "write_kv launch");
  return ok();
}

// Validation and kernel parameters of bsp_prefix_attn for one plan.
static bsp_status_t prefix_params(bsp_plan_s* pl, const void* q, const void* k_pool,
                                  const void* v_pool, float* o_part, float* lse_part,
                                  bsp::PrefixParams& p) {
  bsp_status_t st = check_beam_ready(pl);
  if (st != BSP_OK) return st;
  if (!q || !k_pool || !v_pool || !o_part || !lse_part) return fail(BSP_ERR_ARG, "null pointer");
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(o_part))
    return fail(BSP_ERR_ARG, "q, the pools and o_part must be 16-byte aligned");
  const bsp_layer_desc_t& d = pl->desc;
  p = bsp::PrefixParams{};
  p.q = q;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.o_part = o_part;
  p.lse_part = lse_part;
  p.req = dev_req(pl);
  p.pages = dev_pages(pl);
  p.hdr = dev_header(pl);
  p.B = pl->B;
  p.W = pl->W;
  p.q_len = pl->q_len;
  p.hq = d.num_q_heads;
  p.hkv = d.num_kv_heads;
  p.group = d.num_q_heads / d.num_kv_heads;
  p.page_shift = pl->page_shift;
  p.num_pages = d.num_pages;
  p.n_split = pl->n_split;
  p.split_keys = pl->split_keys;
  p.n_qtiles = (int32_t)ceil_div(pl->rows_per_req, pl->prefix_rpt);
  p.xcd_remap = p.n_qtiles > 1 && (int64_t)p.B * p.hkv * p.n_split % 8 == 0 ? 1 : 0;
  p.causal = d.mask == BSP_MASK_CAUSAL ? 1 : 0;
  p.rows_total = pl->B * pl->W * pl->q_len;
  p.scale = d.sm_scale;
  p.scale_log2e = d.sm_scale * 1.4426950408889634f;
  return BSP_OK;
}

bsp_status_t bsp_prefix_attn(bsp_plan_t pl, const void* q, const void* k_pool, const void* v_pool,
                             float* o_part, float* lse_part, hipStream_t stream) {
  bsp::PrefixParams p{};
  const bsp_status_t st = prefix_params(pl, q, k_pool, v_pool, o_part, lse_part, p);
  if (st != BSP_OK) return st;
  const bsp_layer_desc_t& d = pl->desc;
  return after_launch(pl, bsp::launch_prefix(p, d.dtype, d.head_dim, pl->prefix_rpt, stream),
                      "prefix launch", stream);
}

bsp_status_t bsp_cached_decode(bsp_plan_t pl, const void* q, const void* k_new, const void* v_new,
                               int64_t new_row_stride, const int32_t* slots_d, void* k_pool,
                               void* v_pool, float* o_part, float* lse_part, void* o_out,
                               float* lse_out, hipStream_t stream) {
  bsp::PrefixParams p{};
  bsp_status_t st = prefix_params(pl, q, k_pool, v_pool, o_part, lse_part, p);
  if (st != BSP_OK) return st;
  const bsp_layer_desc_t& d = pl->desc;
  if (d.key_bucket <= 0 || pl->q_len != 1 || pl->W != 1)
    return fail(BSP_ERR_UNSUPPORTED,
                "bsp_cached_decode needs a cached-prefix plan with q_len 1 and one beam");
  if (d.dtype == BSP_F32)
    return fail(BSP_ERR_UNSUPPORTED, "bsp_cached_decode runs bf16/f16; use the separate calls for f32");
  if (pl->prefix_rpt != 64 || pl->rows_per_req > 64 ||
      !bsp::cached_decode_supported(d.num_q_heads / d.num_kv_heads, d.head_dim))
    return fail(BSP_ERR_UNSUPPORTED,
                "bsp_cached_decode takes at most 64 query rows per KV head and query heads per "
                "KV head x head_dim / 4 at most 256");
  if ((int64_t)pl->n_split * pl->rows_total * d.num_q_heads * d.head_dim * 4 > (int64_t)UINT32_MAX)
    return fail(BSP_ERR_UNSUPPORTED,
                "bsp_cached_decode addresses its partial states with 32-bit offsets: %d chunks x "
                "%d rows x %d heads x %d floats is too many",
                pl->n_split, pl->rows_total, d.num_q_heads, d.head_dim);
  if (!k_new || !v_new || !slots_d || !o_out) return fail(BSP_ERR_ARG, "null pointer");
  if (new_row_stride < (int64_t)d.num_kv_heads * d.head_dim || new_row_stride % 8 != 0)
    return fail(BSP_ERR_ARG, "new_row_stride %lld must be >= %d and a multiple of 8",
                (long long)new_row_stride, d.num_kv_heads * d.head_dim);
  if (!aligned16(k_new) || !aligned16(v_new) || (reinterpret_cast<uintptr_t>(o_out) & 7u) != 0)
    return fail(BSP_ERR_ARG, "k_new and v_new must be 16-byte aligned, o_out 8-byte");
  bsp::FusedParams f{};
  f.k_new = k_new;
  f.v_new = v_new;
  f.new_stride = new_row_stride;
  f.k_pool_w = k_pool;
  f.v_pool_w = v_pool;
  f.o_out = o_out;
  f.lse_out = lse_out;
  f.split_count = reinterpret_cast<int32_t*>(static_cast<char*>(pl->ws_d) + pl->split_count_off);
  f.new_slots = slots_d;
  return after_launch(pl, bsp::launch_cached_decode(p, f, d.dtype, d.head_dim, stream),
                      "cached decode launch", stream);
}

bsp_status_t bsp_cached_decode_merge(bsp_plan_t pl, const void* q, const void* k_new,
                                     const void* v_new, int64_t new_row_stride,
                                     const int32_t* slots_d, void* k_pool, void* v_pool,
                                     const float* o_part, const float* lse_part, void* o_out,
                                     float* lse_out, hipStream_t stream) {
  bsp::PrefixParams p{};
  bsp_status_t st = prefix_params(pl, q, k_pool, v_pool, const_cast<float*>(o_part),
                                  const_cast<float*>(lse_part), p);
  if (st != BSP_OK) return st;
  const bsp_layer_desc_t& d = pl->desc;
  if (d.key_bucket <= 0 || pl->q_len != 1 || pl->W != 1)
    return fail(BSP_ERR_UNSUPPORTED,
                "bsp_cached_decode_merge needs a cached-prefix plan with q_len 1 and one beam");
  if (d.dtype == BSP_F32)
    return fail(BSP_ERR_UNSUPPORTED,
                "bsp_cached_decode_merge runs bf16/f16; use the separate calls for f32");
  if (!k_new || !v_new || !slots_d || !o_out) return fail(BSP_ERR_ARG, "null pointer");
  if (new_row_stride < (int64_t)d.num_kv_heads * d.head_dim || new_row_stride % 8 != 0)
    return fail(BSP_ERR_ARG, "new_row_stride %lld must be >= %d and a multiple of 8",
                (long long)new_row_stride, d.num_kv_heads * d.head_dim);
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(BSP_ERR_ARG, "k_new and v_new must be 16-byte aligned");
  bsp::MergeRowParams m{};
  m.rows = pl->B;
  m.hq = d.num_q_heads;
  m.hkv = d.num_kv_heads;
  m.d = d.head_dim;
  m.n_parts = pl->n_split;
  m.o_parts = o_part;
  m.lse_parts = lse_part;
  m.o_stride = (int64_t)pl->B * d.num_q_heads * d.head_dim;
  m.lse_stride = (int64_t)pl->B * d.num_q_heads;
  m.q = q;
  m.k_new = k_new;
  m.v_new = v_new;
  m.new_stride = new_row_stride;
  m.slots = slots_d;
  m.k_pool = k_pool;
  m.v_pool = v_pool;
  m.page_shift = pl->page_shift;
  m.num_pages = d.num_pages;
  m.scale = d.sm_scale;
  m.o_out = o_out;
  m.lse_out = lse_out;
  m.hdr = p.hdr;
  return after_launch(pl, bsp::launch_merge_row(m, d.dtype, stream), "cached decode merge launch",
                      stream);
}

bsp_status_t bsp_prefix_attn_two(bsp_plan_t a, bsp_plan_t b, const void* q, const void* k_pool,
                                 const void* v_pool, float* o_part_a, float* lse_part_a,
                                 float* o_part_b, float* lse_part_b, hipStream_t stream) {
  if (a == nullptr || b == nullptr) return fail(BSP_ERR_ARG, "null plan");
  if (a == b) return fail(BSP_ERR_ARG, "bsp_prefix_attn_two needs two plans");
  bsp::PrefixParams pa{}, pb{};
  bsp_status_t st = prefix_params(a, q, k_pool, v_pool, o_part_a, lse_part_a, pa);
  if (st != BSP_OK) return st;
  st = prefix_params(b, q, k_pool, v_pool, o_part_b, lse_part_b, pb);
  if (st != BSP_OK) return st;
  const bsp_layer_desc_t& da = a->desc;
  const bsp_layer_desc_t& db = b->desc;
  if (da.dtype != db.dtype || da.head_dim != db.head_dim || da.num_q_heads != db.num_q_heads ||
      da.num_kv_heads != db.num_kv_heads || a->B * a->W * a->q_len != b->B * b->W * b->q_len)
    return fail(BSP_ERR_ARG,
                "the two plans need the same dtype, heads, head_dim and query rows");
  if (da.dtype != BSP_F32 && a->prefix_rpt == 64 && b->prefix_rpt == 64) {
    st = after_launch(a, bsp::launch_prefix_two(pa, pb, da.dtype, da.head_dim, stream),
                      "two-plan prefix launch", stream);
    if (st == BSP_OK && b->check_mode) st = bsp_check(b, stream);
    return st;
  }
  // other tile heights: one launch per plan
  st = after_launch(a, bsp::launch_prefix(pa, da.dtype, da.head_dim, a->prefix_rpt, stream),
                    "prefix launch", stream);
  if (st != BSP_OK) return st;
  return after_launch(b, bsp::launch_prefix(pb, db.dtype, db.head_dim, b->prefix_rpt, stream),
                      "prefix launch", stream);
}

}  // extern "C"

namespace {

// Validation and kernel parameters of the fused beam step (bsp_decode_step).
bsp_status_t decode_params(bsp_plan_s* pl, const void* q, const void* k_new, const void* v_new,
                           int64_t new_row_stride, void* k_pool, void* v_pool,
                           const int32_t* block_tables_d, const int32_t* cache_indirection_d,
                           void* o_out, float* lse_out, bsp::PrefixParams& p,
                           bsp::FusedParams& f) {
  bsp_status_t st = check_beam_ready(pl);
  if (st != BSP_OK) return st;
  const bsp_layer_desc_t& d = pl->desc;
  if (d.dtype == BSP_F32)
    return fail(BSP_ERR_UNSUPPORTED, "bsp_decode_step runs bf16/f16; use the separate calls for f32");
  if (pl->q_len != 1) return fail(BSP_ERR_UNSUPPORTED, "bsp_decode_step needs q_len == 1");
  if (d.key_bucket > 0) return fail(BSP_ERR_UNSUPPORTED, "bsp_decode_step is beam mode only");
  if (d.kv_split != 0) return fail(BSP_ERR_UNSUPPORTED, "bsp_decode_step takes no kv_split");
  if (!q || !k_new || !v_new || !k_pool || !v_pool || !block_tables_d || !cache_indirection_d ||
      !o_out)
    return fail(BSP_ERR_ARG, "null pointer");
  const int vec = 8;  // 16 bytes of 2-byte elements
  if (new_row_stride < (int64_t)d.num_kv_heads * d.head_dim || new_row_stride % vec != 0)
    return fail(BSP_ERR_ARG, "new_row_stride %lld must be >= %d and a multiple of %d",
                (long long)new_row_stride, d.num_kv_heads * d.head_dim, vec);
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) ||
      !aligned16(v_pool) || !aligned16(o_out))
    return fail(BSP_ERR_ARG, "q, k_new, v_new, the pools and o_out must be 16-byte aligned");
  p = bsp::PrefixParams{};
  p.q = q;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.req = dev_req(pl);
  p.fitems = reinterpret_cast<const bsp::FusedItem*>(static_cast<char*>(pl->ws_d) + pl->fitems_off);
  p.pages = dev_pages(pl);
  p.hdr = dev_header(pl);
  p.B = pl->B;
  p.W = pl->W;
  p.q_len = 1;
  p.hq = d.num_q_heads;
  p.hkv = d.num_kv_heads;
  p.group = d.num_q_heads / d.num_kv_heads;
  p.page_shift = pl->page_shift;
  p.num_pages = d.num_pages;
  p.n_split = 1;
  p.split_keys = 0;
  const int rows_per_tile = bsp::prefix_rows_per_tile(d.dtype, d.head_dim, pl->rows_per_req);
  p.n_qtiles = (int32_t)ceil_div(pl->rows_per_req, rows_per_tile);
  // the grid is (item, KV head, query tile): the remap is a bijection when
  // items x KV heads is a multiple of 8
  p.xcd_remap = p.n_qtiles > 1 && (int64_t)pl->n_fitems * p.hkv % 8 == 0 ? 1 : 0;
  p.causal = 0;
  p.rows_total = pl->B * pl->W;
  p.scale = d.sm_scale;
  p.scale_log2e = d.sm_scale * 1.4426950408889634f;
  f = bsp::FusedParams{};
  f.k_new = k_new;
  f.v_new = v_new;
  f.new_stride = new_row_stride;
  f.k_pool_w = k_pool;
  f.v_pool_w = v_pool;
  f.block_tables = block_tables_d;
  f.ci = cache_indirection_d;
  f.max_blocks = pl->max_blocks;
  f.max_seq_len = pl->max_seq_len;
  f.o_out = o_out;
  f.lse_out = lse_out;
  f.split_count = nullptr;
  f.split_part = nullptr;
  f.part_floats = pl->part_floats;
  if (pl->n_slots > 0) {
    char* ws = static_cast<char*>(pl->ws_d);
    f.split_count = reinterpret_cast<int32_t*>(ws + pl->split_count_off);
    f.split_part = reinterpret_cast<float*>(ws + pl->split_part_off);
  }
  // output rows (and their lse) plus the current tokens' K and V rows
  const int64_t e = elem_bytes(d.dtype);
  const int64_t rows = (int64_t)pl->B * pl->W;
  const int64_t writes = rows * d.num_q_heads * (d.head_dim * e + (lse_out ? 4 : 0)) +
                         rows * d.num_kv_heads * d.head_dim * e * 2;
  f.stream_out = writes <= bsp::kStreamOutBytes ? 1 : 0;
  return BSP_OK;
}

// Validation and kernel parameters of the context prefill (bsp_prefill_attn).
bsp_status_t prefill_params(bsp_plan_s* pl, const void* q, const void* k_pool, const void* v_pool,
                            void* o_out, float* lse_out, bsp::PrefixParams& p,
                            bsp::FusedParams& f) {
  bsp_status_t st = check_device_ready(pl);
  if (st != BSP_OK) return st;
  if (!pl->prefill)
    return fail(BSP_ERR_STALE_PLAN, "plan holds no prefill step: call bsp_plan_prefill");
  const bsp_layer_desc_t& d = pl->desc;
  if (d.dtype == BSP_F32) return fail(BSP_ERR_UNSUPPORTED, "bsp_prefill_attn is bf16/f16 only");
  if (!q || !k_pool || !v_pool || !o_out) return fail(BSP_ERR_ARG, "null pointer");
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(o_out))
    return fail(BSP_ERR_ARG, "q, the pools and o_out must be 16-byte aligned");
  p = bsp::PrefixParams{};
  p.q = q;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.req = dev_req(pl);
  p.pages = dev_pages(pl);
  p.hdr = dev_header(pl);
  p.items = reinterpret_cast<const int32_t*>(static_cast<char*>(pl->ws_d) + pl->items_off);
  p.B = pl->B;
  p.W = 1;
  p.q_len = 1;
  p.hq = d.num_q_heads;
  p.hkv = d.num_kv_heads;
  p.group = d.num_q_heads / d.num_kv_heads;
  p.page_shift = pl->page_shift;
  p.num_pages = d.num_pages;
  p.n_split = 1;
  p.split_keys = 0;
  p.n_qtiles = 1;
  p.causal = 1;
  p.rows_total = pl->rows_total;
  p.scale = d.sm_scale;
  p.scale_log2e = d.sm_scale * 1.4426950408889634f;
  f = bsp::FusedParams{};
  f.o_out = o_out;
  f.lse_out = lse_out;
  return BSP_OK;
}

}  // namespace

extern "C" {

bsp_status_t bsp_decode_step(bsp_plan_t pl, const void* q, const void* k_new, const void* v_new,
                             int64_t new_row_stride, void* k_pool, void* v_pool,
                             const int32_t* block_tables_d, const int32_t* cache_indirection_d,
                             void* o_out, float* lse_out, hipStream_t stream) {
  bsp::PrefixParams p;
  bsp::FusedParams f;
  const bsp_status_t st = decode_params(pl, q, k_new, v_new, new_row_stride, k_pool, v_pool,
                                        block_tables_d, cache_indirection_d, o_out, lse_out, p, f);
  if (st != BSP_OK) return st;
  const bsp_layer_desc_t& d = pl->desc;
  return after_launch(pl,
                      bsp::launch_decode_step(p, f, d.dtype, d.head_dim, pl->rows_per_req,
                                              pl->n_fitems, pl->tail_pad, stream),
                      "decode step launch", stream);
}

bsp_status_t bsp_debug_fused_slots(bsp_plan_t pl, const void* q, const void* k_new,
                                   const void* v_new, int64_t new_row_stride, void* k_pool,
                                   void* v_pool, const int32_t* block_tables_d,
                                   const int32_t* cache_indirection_d, void* o_out,
                                   int32_t* slots_out_d, hipStream_t stream) {
  bsp::PrefixParams p;
  bsp::FusedParams f;
  const bsp_status_t st = decode_params(pl, q, k_new, v_new, new_row_stride, k_pool, v_pool,
                                        block_tables_d, cache_indirection_d, o_out, nullptr, p, f);
  if (st != BSP_OK) return st;
  if (slots_out_d == nullptr) return fail(BSP_ERR_ARG, "null slots_out");
  const bsp_layer_desc_t& d = pl->desc;
  if (!bsp::decode_uses_slot_table(d.head_dim, pl->rows_per_req, pl->W,
                                   d.num_q_heads / d.num_kv_heads, pl->tail_pad))
    return fail(BSP_ERR_UNSUPPORTED,
                "this plan's tails are gathered key by key, without the LDS slot table");
  f.dump_slots = slots_out_d;
  f.dump_pad = std::max(pl->tail_pad, 1);
  return after_launch(pl,
                      bsp::launch_decode_step(p, f, d.dtype, d.head_dim, pl->rows_per_req,
                                              pl->n_fitems, pl->tail_pad, stream),
                      "fused slot-table dump launch", stream);
}

bsp_status_t bsp_prefill_attn(bsp_plan_t pl, const void* q, const void* k_pool, const void* v_pool,
                              void* o_out, float* lse_out, hipStream_t stream) {
  bsp::PrefixParams p;
  bsp::FusedParams f;
  const bsp_status_t st = prefill_params(pl, q, k_pool, v_pool, o_out, lse_out, p, f);
  if (st != BSP_OK) return st;
  const bsp_layer_desc_t& d = pl->desc;
  return after_launch(pl, bsp::launch_prefill(p, f, d.dtype, d.head_dim, pl->prefill_mb, pl->n_items, stream),
                      "prefill launch", stream);
}

bsp_status_t bsp_mixed_step(bsp_plan_t gen, bsp_plan_t ctx, const void* q, const void* k_new,
                            const void* v_new, int64_t new_row_stride, void* k_pool, void* v_pool,
                            const int32_t* block_tables_d, const int32_t* cache_indirection_d,
                            void* o_out, float* lse_out, const void* q_ctx, const void* k_pool_ctx,
                            const void* v_pool_ctx, void* o_ctx, float* lse_ctx,
                            hipStream_t stream) {
  if (gen == nullptr || ctx == nullptr) return fail(BSP_ERR_ARG, "null plan");
  if (gen == ctx) return fail(BSP_ERR_ARG, "a mixed step needs two plans");
  bsp::PrefixParams dp, pp;
  bsp::FusedParams df, pf;
  bsp_status_t st = decode_params(gen, q, k_new, v_new, new_row_stride, k_pool, v_pool,
                                  block_tables_d, cache_indirection_d, o_out, lse_out, dp, df);
  if (st != BSP_OK) return st;
  st = prefill_params(ctx, q_ctx, k_pool_ctx, v_pool_ctx, o_ctx, lse_ctx, pp, pf);
  if (st != BSP_OK) return st;
  const bsp_layer_desc_t& d = gen->desc;
  const bsp_layer_desc_t& dc = ctx->desc;
  if (d.dtype != dc.dtype || d.head_dim != dc.head_dim)
    return fail(BSP_ERR_ARG, "the two plans of a mixed step need the same dtype and head_dim");
  if (bsp::mixed_step_supported(dp, df, d.dtype, d.head_dim, gen->rows_per_req, gen->tail_pad,
                                ctx->prefill_mb)) {
    const hipError_t e =
        bsp::launch_mixed_step(dp, df, pp, pf, d.dtype, d.head_dim, ctx->n_items, stream);
    st = after_launch(gen, e, "mixed step launch", stream);
    if (st == BSP_OK && ctx->check_mode) st = bsp_check(ctx, stream);
    return st;
  }
  // otherwise the context phase, then the beam step, on the stream
  st = after_launch(ctx, bsp::launch_prefill(pp, pf, dc.dtype, dc.head_dim, ctx->prefill_mb,
                                             ctx->n_items, stream),
                    "prefill launch", stream);
  if (st != BSP_OK) return st;
  return after_launch(gen,
                      bsp::launch_decode_step(dp, df, d.dtype, d.head_dim, gen->rows_per_req,
                                              gen->n_fitems, gen->tail_pad, stream),
                      "decode step launch", stream);
}

static bsp::TailParams tail_params(const bsp_plan_s* pl, const void* q, const void* k_pool,
                                   const void* v_pool, const int32_t* bt, const int32_t* ci) {
  const bsp_layer_desc_t& d = pl->desc;
  bsp::TailParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = q;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.block_tables = bt;
  p.ci = ci;
  p.req = dev_req(pl);
  p.hdr = dev_header(pl);
  p.B = pl->B;
  p.W = pl->W;
  p.hq = d.num_q_heads;
  p.hkv = d.num_kv_heads;
  p.group = d.num_q_heads / d.num_kv_heads;
  p.page_shift = pl->page_shift;
  p.num_pages = d.num_pages;
  p.max_blocks = pl->max_blocks;
  p.max_seq_len = pl->max_seq_len;
  p.tail_pad = pl->tail_pad;
  p.scale = d.sm_scale;
  p.scale_log2e = d.sm_scale * 1.4426950408889634f;
  return p;
}

bsp_status_t bsp_tail_attn(bsp_plan_t pl, const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* block_tables_d, const int32_t* cache_indirection_d,
                           float* o_tail, float* lse_tail, hipStream_t stream) {
  bsp_status_t st = check_beam_ready(pl);
  if (st != BSP_OK) return st;
  if (pl->q_len != 1) return fail(BSP_ERR_UNSUPPORTED, "tail attention needs q_len == 1");
  if (!q || !k_pool || !v_pool || !block_tables_d || !cache_indirection_d || !o_tail || !lse_tail)
    return fail(BSP_ERR_ARG, "null pointer");
  bsp::TailParams p = tail_params(pl, q, k_pool, v_pool, block_tables_d, cache_indirection_d);
  p.o_tail = o_tail;
  p.lse_tail = lse_tail;
  return after_launch(pl, bsp::launch_tail(p, pl->desc.dtype, pl->desc.head_dim, stream),
                      "tail launch", stream);
}

bsp_status_t bsp_naive_beam_attn(bsp_plan_t pl, const void* q, const void* k_pool,
                                 const void* v_pool, const int32_t* block_tables_d,
                                 const int32_t* cache_indirection_d, void* o_out, float* lse_out,
                                 hipStream_t stream) {
  bsp_status_t st = check_beam_ready(pl);
  if (st != BSP_OK) return st;
  if (pl->q_len != 1) return fail(BSP_ERR_UNSUPPORTED, "naive attention needs q_len == 1");
  if (pl->desc.key_bucket > 0) return fail(BSP_ERR_UNSUPPORTED, "naive attention is beam mode only");
  if (!q || !k_pool || !v_pool || !block_tables_d || !cache_indirection_d || !o_out)
    return fail(BSP_ERR_ARG, "null pointer");
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(BSP_ERR_ARG, "q and the pools must be 16-byte aligned");
  bsp::TailParams p = tail_params(pl, q, k_pool, v_pool, block_tables_d, cache_indirection_d);
  return after_launch(pl,
                      bsp::launch_naive(p, o_out, lse_out, pl->desc.dtype, pl->desc.head_dim, stream),
                      "naive launch", stream);
}

bsp_status_t bsp_merge(int32_t rows, int32_t heads, int32_t head_dim, int32_t n_parts,
                       const float* o_parts, const float* lse_parts, int64_t o_part_stride,
                       int64_t lse_part_stride, void* o_out, int32_t out_dtype, float* lse_out,
                       hipStream_t stream) {
  if (rows < 0 || heads <= 0 || head_dim <= 0 || head_dim % 4 != 0 || n_parts <= 0)
    return fail(BSP_ERR_ARG, "bad merge sizes (rows %d heads %d head_dim %d parts %d)", rows, heads,
                head_dim, n_parts);
  if (out_dtype != BSP_F32 && out_dtype != BSP_F16 && out_dtype != BSP_BF16)
    return fail(BSP_ERR_DTYPE, "out_dtype %d is not one of f32, f16, bf16", out_dtype);
  if (rows == 0) return ok();
  if (!o_parts || !lse_parts || !o_out) return fail(BSP_ERR_ARG, "null pointer");
  const int64_t o_need = (int64_t)rows * heads * head_dim, l_need = (int64_t)rows * heads;
  if (n_parts > 1 && (o_part_stride < o_need || lse_part_stride < l_need))
    return fail(BSP_ERR_ARG, "part strides smaller than one part");
  if (!aligned16(o_parts) || o_part_stride % 4 != 0)
    return fail(BSP_ERR_ARG, "o_parts must be 16-byte aligned with a stride multiple of 4");
  bsp::MergeParams p;
  p.rows = rows;
  p.heads = heads;
  p.d = head_dim;
  p.n_parts = n_parts;
  p.o_parts = o_parts;
  p.lse_parts = lse_parts;
  p.o_stride = o_part_stride;
  p.lse_stride = lse_part_stride;
  p.o_out = o_out;
  p.lse_out = lse_out;
  const hipError_t e = bsp::launch_merge(p, out_dtype, stream);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return ok();
}

bsp_status_t bsp_check(bsp_plan_t pl, hipStream_t stream) {
  if (pl == nullptr) return fail(BSP_ERR_ARG, "null plan");
  if (pl->host_only || pl->ws_d == nullptr) return ok();
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  DevHeader h;
  e = hipMemcpy(&h, pl->ws_d, sizeof(h), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy (error word)");
  if (h.error_bits == 0) return ok();
  DevHeader zero;
  std::memset(&zero, 0, sizeof(zero));
  e = hipMemcpy(pl->ws_d, &zero, sizeof(zero), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy (clear error word)");
  return fail(BSP_ERR_DEVICE_INDEX,
              "kernels skipped %d out-of-range index reads/writes (bits 0x%x: 1 prompt page, "
              "2 cache_indirection parent, 4 tail page, 8 write slot); first value %d",
              h.fault_count, h.error_bits, h.first_value);
}

bsp_status_t bsp_debug_plan_tables(bsp_plan_t pl, int32_t* indptr_h, int32_t* pages_h,
                                   int32_t* n_keys_h, int32_t* valid_h, int32_t* tail_h) {
  if (pl == nullptr) return fail(BSP_ERR_ARG, "null plan");
  if (!pl->planned) return fail(BSP_ERR_STALE_PLAN, "plan has no valid step");
  for (int b = 0; b < pl->B; ++b) {
    const ReqInfo& r = pl->h_req[b];
    if (indptr_h) indptr_h[b] = r.page_off;
    if (n_keys_h) n_keys_h[b] = r.n_keys;
    if (valid_h) valid_h[b] = r.valid;
    if (tail_h) tail_h[b] = r.tail;
  }
  if (indptr_h) indptr_h[pl->B] = (int32_t)pl->h_pages.size();
  if (pages_h && !pl->h_pages.empty())
    std::memcpy(pages_h, pl->h_pages.data(), sizeof(int32_t) * pl->h_pages.size());
  return ok();
}

bsp_status_t bsp_debug_plan_items(bsp_plan_t pl, int32_t* n_items_h, int32_t* items_h) {
  if (pl == nullptr || n_items_h == nullptr) return fail(BSP_ERR_ARG, "null pointer");
  if (!pl->planned) return fail(BSP_ERR_STALE_PLAN, "plan has no valid step");
  *n_items_h = pl->n_fitems;
  if (items_h != nullptr)
    for (int i = 0; i < pl->n_fitems; ++i) {
      const bsp::FusedItem& it = pl->h_fitems[i];
      items_h[4 * i] = it.b;
      items_h[4 * i + 1] = it.k_lo;
      items_h[4 * i + 2] = it.k_hi;
      items_h[4 * i + 3] = it.parts;
    }
  return ok();
}

bsp_status_t bsp_debug_tail_slots(bsp_plan_t pl, const int32_t* block_tables_d,
                                  const int32_t* cache_indirection_d, int32_t* slots_d,
                                  hipStream_t stream) {
  bsp_status_t st = check_beam_ready(pl);
  if (st != BSP_OK) return st;
  if (!block_tables_d || !cache_indirection_d || !slots_d) return fail(BSP_ERR_ARG, "null pointer");
  bsp::TailParams p = tail_params(pl, nullptr, nullptr, nullptr, block_tables_d, cache_indirection_d);
  p.slots_out = slots_d;
  return after_launch(pl, bsp::launch_tail_slots(p, stream), "tail slots launch", stream);
}

}  // extern "C"
