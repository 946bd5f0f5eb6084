// Shared-key ("prefix") attention: every query row of a request against the
// request's shared keys, read once per request and KV head.
//
// The prompt is attended once per request with all beams' query rows together
// (TensorRT-LLM PR #21738, "Add opt-in cascade attention for wide beam search
// on KVCM V2", Description: Solution; the FA4 commit feeds one group of
// beam_width queries per request). With W beams and G query heads per KV head
// that is M = W * G rows against the same keys, a real dense contraction, so
// bf16/f16 run on the gfx950 matrix cores (v_mfma_f32_16x16x32_{bf16,f16}).
//
// Work item: (request b, KV head g, key split, query-row tile). A workgroup is
// 4 waves; each wave owns 16*MB query rows. Keys stream through LDS in tiles
// of KT rows (K and V, row stride padded by 16 bytes); the next tile's global
// loads are issued into registers before the current tile is computed.
//
// Products are taken transposed so that queries sit on the MFMA "n" index
// (lane % 16) in both of them:
//   S^T[key][query] = sum_d K[key][d] * Q[query][d]     A = K (LDS), B = Q^T (registers)
//   O^T[d][query]  += sum_key V[key][d] * P[query][key] A = V^T (LDS), B = P^T
// The 16x16 accumulator layout puts S^T[4*(lane/16)+e][lane%16] in lane
// `lane`, element e; those are exactly the (query, key) pairs the lane must
// supply as the B operand of the second product, so P^T never crosses lanes,
// and O^T's rows per query live in the same lane as that query's softmax
// statistics. Both operands of each product enumerate the contraction index
// in the same per-lane order, so the result does not depend on how the
// hardware orders the 32-wide contraction inside an instruction.
//
// Online softmax (running max m and sum l per query row, rescaling O when m
// grows) is taken in base 2 on the raw dot products: p = 2^((s - m) * scale *
// log2 e). f32 runs a vector-ALU kernel (one wave per query row).
#include <climits>

#include "bsp_internal.h"
#include "device_common.h"
#include "tile_index.h"

namespace bsp {

template <typename T> struct Mfma;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// mma: 16x16 output, 32-long contraction (8 elements per lane);
// mma16: 16-long contraction (4 elements per lane), operands as raw 16-bit words.
template <> struct Mfma<__bf16> {
  using V8 = bf16x8;
  static __device__ __forceinline__ f32x4 mma(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
  }
};
template <> struct Mfma<_Float16> {
  using V8 = f16x8;
  static __device__ __forceinline__ f32x4 mma(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
};

struct WorkItem {
  int b, g, split, qt;
  int k_lo, k_hi;  // key range of this item (keys >= k_hi are never read)
};

// Page ids of one request are staged in LDS in windows of this many pages, so
// issuing a tile's loads never waits on a global page-id load.
constexpr int kPageWin = 1024;
// Resolved tail slots of the fused step, per (beam of this query tile, tail
// position); larger tails are resolved on the fly.
constexpr int kTailSlots = 3072;
// Lazy rescaling threshold of the online softmax, in base-2 exponent units.
constexpr float kLazyLog2 = 8.f;

// Wait until at most N vector-memory operations of this wave are in flight
// (vmcnt only; LDS and export counters unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// Wait until this wave's LDS reads have completed (lgkmcnt 0, other counters free).
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// 16-byte direct global-to-LDS load (one per lane; a wave fills 1 KB at
// `lds_dst` + 16 * lane). Issued through inline asm so that the compiler does
// not see an LDS-writing load: it would otherwise wait for every load in
// flight before each LDS read. Ordering is explicit instead: wait_vmcnt()
// for the tile, then a workgroup barrier, before any wave reads it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void* src, void* lds_dst) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)lds_dst);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(m0), "v"(src) : "memory", "m0");
}
// The same with a wave-uniform 64-bit base and a per-lane 32-bit byte offset
// (the scalar-base form of the load: no per-lane 64-bit address arithmetic).
__device__ __forceinline__ void lds_dma16_s(const void* base, unsigned voff, void* lds_dst) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)lds_dst);
  // readfirstlane yields a signed int: widen through unsigned, or a low word
  // with bit 31 set would be sign-extended over the high word.
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint64_t lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)b);
  const uint64_t hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(b >> 32));
  const uint64_t sb = lo | (hi << 32);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(m0), "v"(voff), "s"(sb) : "memory", "m0");
}
#pragma clang diagnostic pop

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Four consecutive keys' values of one column, transposed across 16 lanes:
// lane (4e + q) of each 16-lane group reads 4 values of row `row_e` at column
// `col4`; afterwards lane i holds the values of column (col4 base + i) of the
// 4 rows of its group.
__device__ __forceinline__ s16x4 lds_read_tr(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}

// Variants whose row blocks need more than half a SIMD's registers run one
// workgroup per CU (accumulators may then live in AGPRs).
template <int D, int MB>
constexpr int prefix_min_blocks() { return MB * D >= 512 ? 1 : 2; }

// Tail slot encoding: >= 0 pool row index ((page * Hkv + g) * page_size + row);
// -1 an invalid index (skipped); <= -2 the current token of beam (-entry - 2),
// read from the new-token rows instead of the pool.
__device__ __forceinline__ int32_t resolve_fused_slot(const PrefixParams& p, const FusedParams& f,
                                                      int b, int kk, int g, int j, int jcur) {
  const int32_t src = f.ci[((int64_t)b * p.W + kk) * f.max_seq_len + j];
  if (src < 0 || src >= p.W) {
    record_fault(&p.hdr->error_bits, &p.hdr->fault_count, &p.hdr->first_value, kErrTailParent, src);
    return -1;
  }
  if (j == jcur) return -2 - src;
  const int32_t page = f.block_tables[((int64_t)b * p.W + src) * f.max_blocks + (j >> p.page_shift)];
  if (page < 0 || page >= p.num_pages) {
    record_fault(&p.hdr->error_bits, &p.hdr->fault_count, &p.hdr->first_value, kErrTailPage, page);
    return -1;
  }
  return ((page * p.hkv + g) << p.page_shift) + (j & ((1 << p.page_shift) - 1));
}

// MODE 0: bsp_prefix_attn (fp32 partial state per key split).
// MODE 1 and 2: bsp_decode_step, one launch per layer step: the workgroup of
// (request, KV head, query tile) also writes its beams' current tokens and
// attends each beam's tail (gathered through cache_indirection) in the same
// online softmax as the shared keys, then writes the final output in the
// storage dtype. MODE 1 resolves the tail slots into an LDS table and, after
// the shared keys, each wave streams its own beams' tail rows through its
// quarter of the then idle tile ring; MODE 2, for tails too long for that
// table, gathers them key by key afterwards.
// MODE 3: bsp_prefill_attn, the context requests of a mixed step: ragged query
// rows packed per request, each row attending the request's cached rows and,
// causally, the chunk's rows up to its own; work items (request, query tile)
// come from the plan's list and key tiles past a tile's last visible key are
// never loaded; the output is written in the storage dtype.
// MODE 5: MODE 0 for a one-row cached-prefix decode, with the chunks' partial
// states merged with this call's row by the last chunk to finish (one launch).
// MODE 4: a mixed step in one launch: each workgroup is either a MODE 1 item
// of the beam step or a MODE 3 item of the context requests (`pre`), with
// that part's parameters.
// The beam step (MODES 1, 2 and the beam-step items of 4) takes its work
// items from the plan's list (FusedItem), longest first. An item covers all of
// a request's prompt, or one chunk of it when the plan split the prompt; then
// the workgroup leaves its partial state in its slot and counts itself on the
// request's counter, and only the last of the request's workgroups (per KV
// head and query tile) to arrive merges the other chunks' states and
// finishes the request (tails, output, current-token write). No workgroup
// ever waits for another.
template <typename T, int D, int MB, int KT, int NST, int MODE>
__device__ __forceinline__ void prefix_body(PrefixParams p, FusedParams f, int block, bool pre) {
  // FUSED / PREFILL: the workgroup may be a beam-step / context item; `fused`
  // and `is_pre` say which one it is.
  constexpr bool FUSED = MODE == 1 || MODE == 2 || MODE == 4;
  constexpr bool PREFILL = MODE == 3 || MODE == 4;
  constexpr bool TAILS1 = MODE == 1 || MODE == 4;  // tails through the LDS slot table
  const bool is_pre = MODE == 3 || (MODE == 4 && pre);
  const bool fused = FUSED && !is_pre;
  static_assert(MODE != 4 || MB == 1, "mixed steps take one query block per wave");
  using V8 = typename Mfma<T>::V8;
  using TG = TileGeom<(int)sizeof(T), D, KT, NST>;  // LDS and global offsets (tile_index.h)
  constexpr int NDS = D / 32;                       // contraction steps of S^T
  constexpr int NDB = D / 16;                       // 16-row blocks of O^T
  constexpr int NKB = KT / 16;                      // 16-key blocks of S^T per tile
  constexpr int NS2 = KT / 32;                      // contraction steps of O^T per tile
  constexpr int CPR = D / 8;                        // 16-byte chunks per key row
  constexpr int TILE = KT * D;                      // elements of K (or V) per tile
  constexpr int NI = TILE * (int)sizeof(T) / 4096;  // 1 KB loads per wave for K (and V)
  constexpr int LPT = 2 * NI;                       // vector-memory ops per thread per tile
  static_assert(NI >= 1 && TILE * sizeof(T) % 4096 == 0, "tile must split into 1 KB loads");
  static_assert(NST >= 2 && NST <= 4 && 2 * LPT < 64, "pipeline depth");
  __shared__ __attribute__((aligned(1024))) T lds_kv[NST][2][TILE];
  T* const lds_ring = &lds_kv[0][0][0];  // the ring as one array (TileGeom offsets)
  __shared__ int lds_pages[kPageWin];
  __shared__ int lds_tail[TAILS1 ? kTailSlots : 1];

  // ---- work: one (request or prompt chunk, KV head, key split, query tile) item
  WorkItem w;
  ReqInfo ri;
  int part = 0, parts = 1, slot = -1;  // split requests of the beam step
  {
    int bid = block;
    if (fused) {
      // (item, KV head, query tile), items longest first
      if (p.xcd_remap) {
        // Workgroups are dealt to the 8 XCDs in turn, so block ids 8 apart
        // share an XCD and its L2: the query tiles of one item go there.
        const int lo = bid & 7;
        const int rest = bid >> 3;
        w.qt = rest % p.n_qtiles;
        bid = (rest / p.n_qtiles) * 8 + lo;
      } else {
        w.qt = bid % p.n_qtiles;
        bid /= p.n_qtiles;
      }
      w.g = bid % p.hkv;
      const FusedItem it = p.fitems[bid / p.hkv];
      ri = it.ri;
      w.b = it.b;
      w.k_lo = it.k_lo;
      w.k_hi = it.k_hi;
      w.split = 0;
      part = it.part;
      parts = it.parts;
      slot = it.slot;
    } else if (PREFILL && is_pre) {
      w.g = bid % p.hkv;
      const int item = bid / p.hkv;
      w.b = p.items[2 * item];
      w.qt = p.items[2 * item + 1];
      w.split = 0;
      // keys up to the tile's last row (row r holds chunk position r / group)
      ri = p.req[w.b];
      const int last = min((w.qt + 1) * 64 * MB, ri.tail * p.group) - 1;
      w.k_lo = 0;
      w.k_hi = min(ri.valid, ri.valid - ri.tail + last / p.group + 1);
    } else if (p.causal && p.W == 1) {
      // Causal rows of one sequence: row r is position r / group and sees keys
      // up to n_keys - q_len + r / group, so a tile streams only the keys up to
      // its last row's limit. Tiles go longest first (query tile slowest,
      // descending), so the short ones fill the last round.
      w.g = bid % p.hkv;
      bid /= p.hkv;
      w.split = bid % p.n_split;
      bid /= p.n_split;
      w.b = bid % p.B;
      w.qt = p.n_qtiles - 1 - bid / p.B;
      ri = p.req[w.b];
      const int r_last = min((w.qt + 1) * 64 * MB, p.q_len * p.group) - 1;
      const int lim = min(ri.valid, ri.n_keys - p.q_len + r_last / p.group + 1);
      w.k_lo = p.split_keys > 0 ? w.split * p.split_keys : 0;
      w.k_hi = p.split_keys > 0 ? min(lim, w.k_lo + p.split_keys) : lim;
      if (w.k_hi < w.k_lo) w.k_hi = w.k_lo;
    } else {
      if (p.xcd_remap) {
        const int lo = bid & 7;
        const int rest = bid >> 3;
        w.qt = rest % p.n_qtiles;
        bid = (rest / p.n_qtiles) * 8 + lo;
      } else {
        w.qt = bid % p.n_qtiles;
        bid /= p.n_qtiles;
      }
      w.split = bid % p.n_split;
      bid /= p.n_split;
      w.g = bid % p.hkv;
      w.b = bid / p.hkv;
      ri = p.req[w.b];
      w.k_lo = p.split_keys > 0 ? w.split * p.split_keys : 0;
      w.k_hi = p.split_keys > 0 ? min(ri.valid, w.k_lo + p.split_keys) : ri.valid;
      if (w.k_hi < w.k_lo) w.k_hi = w.k_lo;
    }
  }
  const bool split = fused && parts > 1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform by construction
  const int l16 = lane & 15;
  const int l4 = lane >> 4;

  const int M = is_pre ? ri.tail * p.group : p.W * p.q_len * p.group;
  // Rows per wave: 16 per query block; in the fused step with one block per
  // wave and at most 32 (16) query rows per request, 8 (4) per wave, so that
  // all four waves share the beams' tails instead of two (one) of them. Lanes
  // past a wave's rows are treated like rows past M.
  const int rpw = TAILS1 && !is_pre && MB == 1 && p.n_qtiles == 1 ? (M <= 16 ? 4 : M <= 32 ? 8 : 16) : 16;
  const int row0 = w.qt * (64 * MB) + wave * (rpw * MB);
  const bool wave_active = row0 < M;
  const int row_end = min(M, row0 + rpw * MB);  // this wave's rows: [row0, row_end)
  const int shift = p.page_shift;
  const int pmask = (1 << shift) - 1;

  // ---- fused step: the beams with a row in this query tile, their tail slots
  const int rt = 64 * MB;                       // query rows per workgroup
  const int kb_first = (w.qt * rt) / p.group;   // beams with a row in this tile
  const int kb_last = min(p.W - 1, ((w.qt + 1) * rt - 1) / p.group);
  const int nbt = kb_last - kb_first + 1;
  // MODE 1 tail slots of this tile's beams (slot-table rows u = (beam -
  // kb_first) * n_tail + t), TR per thread at a time: all parent lookups, then
  // all page lookups, then the table entries (the host checked that the table
  // holds them). A workgroup of a split request builds the table only once it
  // knows that it finishes the request.
  constexpr int TR = 4;
  const int n_sl = TAILS1 && fused ? nbt * ri.tail : 0;
  auto sl_parents = [&](int base, int32_t (&src)[TR]) {
#pragma unroll
    for (int i = 0; i < TR; ++i) {
      const int task = base + i * 256 + tid;
      src[i] = -1;
      if (task < n_sl) {
        const int kk = kb_first + task / ri.tail;
        src[i] = f.ci[((int64_t)w.b * p.W + kk) * f.max_seq_len + ri.prefix + task % ri.tail];
      }
    }
  };
  auto sl_pages = [&](int base, const int32_t (&src)[TR], int32_t (&page)[TR]) {
#pragma unroll
    for (int i = 0; i < TR; ++i) {
      const int task = base + i * 256 + tid;
      const int j = ri.prefix + task % max(ri.tail, 1);
      page[i] = -1;
      if (task < n_sl && src[i] >= 0 && src[i] < p.W && j != ri.seq - 1)
        page[i] = f.block_tables[((int64_t)w.b * p.W + src[i]) * f.max_blocks + (j >> shift)];
    }
  };
  auto sl_commit = [&](int base, const int32_t (&src)[TR], const int32_t (&page)[TR]) {
#pragma unroll
    for (int i = 0; i < TR; ++i) {
      const int task = base + i * 256 + tid;
      if (task >= n_sl) continue;
      const int j = ri.prefix + task % ri.tail;
      int32_t e;
      if (src[i] < 0 || src[i] >= p.W) {
        record_fault(&p.hdr->error_bits, &p.hdr->fault_count, &p.hdr->first_value,
                     kErrTailParent, src[i]);
        e = -1;
      } else if (j == ri.seq - 1) {
        e = -2 - src[i];
      } else if (page[i] < 0 || page[i] >= p.num_pages) {
        record_fault(&p.hdr->error_bits, &p.hdr->fault_count, &p.hdr->first_value,
                     kErrTailPage, page[i]);
        e = -1;
      } else {
        e = (int32_t)(pool_row(page[i], p.hkv, w.g, shift, j & pmask, 1));
      }
      lds_tail[task] = e;
    }
  };
  // With one query block per wave the first batch's lookups overlap the start
  // of the prompt stream: parents go out with the queries and the first page
  // ids, pages right after, and the table is written once the prompt is done.
  // (With more blocks the eight registers they hold cost more than the
  // overlap gains: measured at MB = 2, not free at MB = 3.)
  constexpr bool DEFER = MODE == 1 && MB == 1;
  int32_t t_src[TR], t_page[TR];
  auto sl_build = [&](int from) {
    for (int base = from; base < n_sl; base += 256 * TR) {
      sl_parents(base, t_src);
      sl_pages(base, t_src, t_page);
      sl_commit(base, t_src, t_page);
    }
  };
  if constexpr (TAILS1 && !DEFER) {
    if (!split) sl_build(0);
  }

  // ---- query rows of this lane (B operand of S^T), causal limits
  V8 qv[MB][NDS];
  int climit[MB];
#pragma unroll
  for (int qb = 0; qb < MB; ++qb) {
    const int r = row0 + qb * 16 + l16;
    climit[qb] = INT_MAX;
    if (r < row_end) {
      const int hh = r % p.group;
      const int t = r / p.group;
      int64_t qrow;
      if (PREFILL && is_pre) {  // packed rows; chunk position t sees keys up to valid - rows + t
        qrow = ((int64_t)ri.q_off + t) * p.hq + w.g * p.group + hh;
        climit[qb] = ri.valid - ri.tail + t;
      } else {
        const int i = t % p.q_len;
        const int kbeam = t / p.q_len;
        qrow = (((int64_t)w.b * p.W + kbeam) * p.q_len + i) * p.hq + w.g * p.group + hh;
        if (p.causal) climit[qb] = ri.n_keys - p.q_len + i;
      }
      const T* qp = static_cast<const T*>(p.q) + qrow * D + l4 * 8;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) qv[qb][ds] = *reinterpret_cast<const V8*>(qp + ds * 32);
    } else {
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[qb][ds][e] = Traits<T>::from_f(0.f);
      }
    }
  }

  if constexpr (DEFER) {
    if (!split) sl_parents(0, t_src);
  }

  f32x4 oacc[NDB][MB];
  float mrow[MB], lrow[MB];
#pragma unroll
  for (int qb = 0; qb < MB; ++qb) {
    mrow[qb] = -INFINITY;
    lrow[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const T* kpool = static_cast<const T*>(p.k_pool);
  const T* vpool = static_cast<const T*>(p.v_pool);
  const float c2 = p.scale_log2e;
  const int keys_per_win = kPageWin << shift;

  // One tile against the query blocks of this wave, in three parts:
  // s_tile: S^T = K Q^T;
  // softmax_tile: masking (`visible(qb, kk)`, consulted only when `full` is
  //   false) and the online softmax; P^T leaves as the B operand of O^T;
  // o_tile: O^T += V^T P^T.
  // The operands of both products are read from LDS PF ahead of their use,
  // so a read's latency overlaps the matrix instructions of the operands
  // before it (reading each operand right before its use waited one LDS round
  // trip per operand; the compiler keeps what its register budget allows).
  constexpr int PF = MB == 1 ? 4 : MB == 2 ? 2 : 1;
  auto s_tile = [&](const T* lk, f32x4 (&sacc)[NKB][MB]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int qb = 0; qb < MB; ++qb) sacc[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int NOP = NDS * NKB;  // operand i: key block i % NKB, contraction step i / NKB
    auto ld = [&](int i) -> V8 {
      return *reinterpret_cast<const V8*>(&lk[TG::k_read((i % NKB) * 16 + l16, (i / NKB) * 4 + l4)]);
    };
    V8 a[PF + 1];
#pragma unroll
    for (int i = 0; i < PF && i < NOP; ++i) a[i] = ld(i);
#pragma unroll
    for (int i = 0; i < NOP; ++i) {
      if (i + PF < NOP) a[(i + PF) % (PF + 1)] = ld(i + PF);
#pragma unroll
      for (int qb = 0; qb < MB; ++qb)
        sacc[i % NKB][qb] = Mfma<T>::mma(a[i % (PF + 1)], qv[qb][i / NKB], sacc[i % NKB][qb]);
    }
  };

  // A row's reference max m is raised only when the tile's max passes it by
  // more than kLazyLog2 (base-2 units); otherwise O and l keep their scale and
  // the tile's probabilities stay below 2^kLazyLog2, far inside the bf16/f16
  // range. The log-sum-exp is taken against the same m, so the result is that
  // of the exact running-max update.
  const float lazy_keys = kLazyLog2 / c2;  // the lazy threshold in raw score units
  auto softmax_tile = [&](f32x4 (&sacc)[NKB][MB], bool full, auto&& visible, V8 (&pb)[NS2][MB]) {
    if (__builtin_expect(!full, 0)) {  // wave-uniform: only a tile crossing the key bound
      asm volatile("" ::: "memory");     // keep it a branch, not selects on every tile
#pragma unroll
      for (int qb = 0; qb < MB; ++qb)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sacc[kb][qb][e] = visible(qb, kb * 16 + l4 * 4 + e) ? sacc[kb][qb][e] : -INFINITY;
    }
#pragma unroll
    for (int qb = 0; qb < MB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sacc[kb][qb][e]);
      // A row's max passes its reference by more than kLazyLog2 exactly when
      // one of its four lanes' maxima does: each lane tests its own against
      // the row's threshold and the row max across the lanes is taken only
      // on the (rare) rescale. -inf + x stays -inf and compares false, as
      // the difference of two -inf (NaN) did.
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(mx > mrow[qb] + lazy_keys) != 0, 0)) {
        // Keep this a branch: the compiler would otherwise scale O on every
        // tile with alpha = 1.
        asm volatile("" ::: "memory");
        mx = max4x16(mx);
        const float m_new = fmaxf(mrow[qb], mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2((mrow[qb] - m_use) * c2);
        mrow[qb] = m_new;
        lrow[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db][qb] *= alpha;
      }
      const float moff = mrow[qb] == -INFINITY ? 0.f : -mrow[qb] * c2;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pr = fast_exp2(fmaf(sacc[kb][qb][e], c2, moff));
          sacc[kb][qb][e] = pr;
          rs += pr;
        }
      }
      lrow[qb] += rs;
#pragma unroll
      for (int s2 = 0; s2 < NS2; ++s2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pb[s2][qb][e] = Traits<T>::from_f(sacc[2 * s2][qb][e]);
          pb[s2][qb][4 + e] = Traits<T>::from_f(sacc[2 * s2 + 1][qb][e]);
        }
      }
    }
  };

  auto o_tile = [&](const T* lv, const V8 (&pb)[NS2][MB]) {
    constexpr int NOP = NS2 * NDB;  // operand i: key step i / NDB, output block i % NDB
    auto ld = [&](int i) -> V8 {
      const int ra = 32 * (i / NDB) + 4 * l4 + (l16 >> 2);  // row read by this lane (+16 for the upper half)
      // The operand is assembled from whole 32-bit words of the two reads
      // (rows ra and ra + 16 share the swizzle: it depends on the low 4 bits).
      const int off = TG::v_read(ra, (i % NDB) * 16 + 4 * (l16 & 3));
      const u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr(&lv[off]));
      const u32x2 hi = __builtin_bit_cast(u32x2, lds_read_tr(&lv[off + 16 * D]));
      return __builtin_bit_cast(V8, u32x4{lo[0], lo[1], hi[0], hi[1]});
    };
    V8 a[PF + 1];
#pragma unroll
    for (int i = 0; i < PF && i < NOP; ++i) a[i] = ld(i);
#pragma unroll
    for (int i = 0; i < NOP; ++i) {
      if (i + PF < NOP) a[(i + PF) % (PF + 1)] = ld(i + PF);
#pragma unroll
      for (int qb = 0; qb < MB; ++qb)
        oacc[i % NDB][qb] = Mfma<T>::mma(a[i % (PF + 1)], pb[i / NDB][qb], oacc[i % NDB][qb]);
    }
  };

  // With two or more query blocks per wave the prompt loop is rotated: tile
  // t's S^T goes to the matrix cores, then tile t-1's O^T, and tile t's
  // softmax runs on the vector ALU while they execute. Tile t-1 then holds
  // its stage one iteration longer, so one tile fewer is loaded ahead.
  constexpr bool ROT = MB >= 2 && NST >= 4;
  constexpr int AHEAD = ROT ? NST - 2 : NST - 1;  // tiles in flight beyond the one computed

  const int n_tail = fused ? ri.tail : 0;
  // ---- current tokens of this tile's beams: a beam's token is written by the
  // tile holding its first row, 16 bytes per task. Nothing in this launch
  // reads it back from the pool (the tails take the current token from the
  // new-token rows), so the stores go last, where they delay no tile.
  const int kw_lo = (w.qt * rt + p.group - 1) / p.group;
  const int kw_hi = min(p.W, ((w.qt + 1) * rt + p.group - 1) / p.group);
  const int n_tw = fused && n_tail > 0 ? (kw_hi - kw_lo) * CPR : 0;
  auto tw_load = [&](int base, auto& page, auto& kd, auto& vd) {
    constexpr int N = (int)(sizeof(page) / sizeof(int32_t));
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int task = base + i * 256 + tid;
      page[i] = -1;
      if (task < n_tw) {
        const int kk = kw_lo + task / CPR;
        const int64_t src = ((int64_t)w.b * p.W + kk) * f.new_stride + (int64_t)w.g * D + (task % CPR) * 8;
        page[i] = f.block_tables[((int64_t)w.b * p.W + kk) * f.max_blocks + ((ri.seq - 1) >> shift)];
        kd[i] = *reinterpret_cast<const u32x4*>(static_cast<const T*>(f.k_new) + src);
        vd[i] = *reinterpret_cast<const u32x4*>(static_cast<const T*>(f.v_new) + src);
      }
    }
  };
  auto tw_store = [&](int base, const auto& page, const auto& kd, const auto& vd) {
    constexpr int N = (int)(sizeof(page) / sizeof(int32_t));
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int task = base + i * 256 + tid;
      if (task >= n_tw) continue;
      if (page[i] < 0 || page[i] >= p.num_pages) {
        if (task % CPR == 0)
          record_fault(&p.hdr->error_bits, &p.hdr->fault_count, &p.hdr->first_value,
                       kErrTailPage, page[i]);
        continue;
      }
      const int64_t dst = pool_row(page[i], p.hkv, w.g, shift, (ri.seq - 1) & pmask, D) + (task % CPR) * 8;
      // streaming stores (see kStreamOutBytes) at up to two query blocks per
      // wave; at three the register budget does not take the second store path
      // without spilling
      if constexpr (MB <= 2) {
        store_maybe_stream(reinterpret_cast<u32x4*>(static_cast<T*>(f.k_pool_w) + dst), kd[i], f.stream_out != 0);
        store_maybe_stream(reinterpret_cast<u32x4*>(static_cast<T*>(f.v_pool_w) + dst), vd[i], f.stream_out != 0);
      } else {
        *reinterpret_cast<u32x4*>(static_cast<T*>(f.k_pool_w) + dst) = kd[i];
        *reinterpret_cast<u32x4*>(static_cast<T*>(f.v_pool_w) + dst) = vd[i];
      }
    }
  };


  // Where each thread has at most TWE tasks (one or two query blocks per wave,
  // head_dim <= 128, an unsplit request) the rows are loaded in the prologue,
  // beside the queries, in the round trip that ends with the wait before the
  // first tile load (a wait the compiler sees), and held until the end, which
  // then has only the stores; otherwise both go last. (Storing them right
  // after the first tile landed measured slower: the stores then count in the
  // tile waits. So did loading them after the prompt, before the tails.)
  constexpr int TWE = MB == 1 ? 4 : 2;
  constexpr bool TW_EARLY = FUSED && MB <= 2 && D <= 128;
  const bool tw_early = TW_EARLY && !split && n_tw > 0 && n_tw <= 256 * TWE;
  int32_t e_page[TWE];
  u32x4 e_kd[TWE], e_vd[TWE];
  // prefill, and causal rows of one sequence: the smallest causal limit among
  // this wave's rows (its first row); a key tile at or below it needs no mask
  const bool causal1 = !FUSED && !is_pre && p.causal && p.W == 1;
  const int c_first = is_pre ? ri.valid - ri.tail + row0 / p.group
                             : causal1 ? ri.n_keys - p.q_len + row0 / p.group : 0;
  const int win_first = w.k_lo / keys_per_win;
  const int n_win = w.k_hi > w.k_lo ? (w.k_hi - 1) / keys_per_win - win_first + 1 : 0;

  // Page ids of one window of the request's keys into LDS.
  auto fill_pages = [&](int wi) {
    const int w0 = (win_first + wi) * keys_per_win;
    const int pg0 = w0 >> shift;
    const int npg = ((min(w.k_hi, w0 + keys_per_win) - 1) >> shift) - pg0 + 1;
    for (int i = tid; i < npg; i += 256) {
      int32_t page = p.pages[ri.page_off + pg0 + i];
      if (page < 0 || page >= p.num_pages) {  // the plan validated these; flag corruption
        record_fault(&p.hdr->error_bits, &p.hdr->fault_count, &p.hdr->first_value,
                     kErrPrefixPage, page);
        page = 0;
      }
      lds_pages[i] = page;
    }
  };
  if constexpr (TW_EARLY) {
    if (tw_early) tw_load(0, e_page, e_kd, e_vd);
  }
  if constexpr (DEFER) {
    if (n_win > 0) fill_pages(0);
    // The queries, the tail parents and the first page ids are complete
    // before any tile load is issued (the compiler does not count the
    // inline-asm tile loads, so a wait it placed later for one of these
    // registers would also wait for every tile in flight). The tail page
    // lookups then stay in flight beside the tiles; they are used after the
    // prompt, when everything has landed.
    wait_vmcnt<0>();
    if (!split) sl_pages(0, t_src, t_page);
  }

  for (int wi = 0; wi < n_win; ++wi) {
    const int w0 = (win_first + wi) * keys_per_win;
    const int seg_lo = max(w.k_lo, w0);
    const int seg_hi = min(w.k_hi, w0 + keys_per_win);
    const int pg0 = w0 >> shift;
    if (!DEFER || wi > 0) {
      __syncthreads();  // every wave is done with the previous window
      fill_pages(wi);
      // also the queries (first window): see above
      wait_vmcnt<0>();
    }
    __syncthreads();
    const int ntp = (seg_hi - seg_lo + KT - 1) / KT;
    const int nt = ntp;

    // Issue the direct-to-LDS loads of one tile into one stage.
    auto issue = [&](int tile, int stage) {
      const int t0 = seg_lo + tile * KT;
      if ((t0 & pmask) + KT <= pmask + 1) {
        // The tile lies in one page: one scalar base per pool, and each lane
        // adds its fixed offset (rows past the key range re-read row t0).
        const int page = __builtin_amdgcn_readfirstlane(lds_pages[window_slot(t0, shift, pg0)]);
        const int64_t base = pool_row(page, p.hkv, w.g, shift, t0 & pmask, D);
        const T* kb = kpool + base;
        const T* vb = vpool + base;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int r = TG::load_row(wave, i, lane);
          const int c = TG::load_chunk(wave, i, lane);
          const unsigned voff = (unsigned)(((t0 + r < seg_hi ? r : 0) * D + c * 8) * (int)sizeof(T));
          lds_dma16_s(kb, voff, &lds_ring[TG::ring_dst(stage, 0, wave, i)]);
          lds_dma16_s(vb, voff, &lds_ring[TG::ring_dst(stage, 1, wave, i)]);
        }
        return;
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int r = TG::load_row(wave, i, lane);
        const int c = TG::load_chunk(wave, i, lane);
        int j = t0 + r;
        if (j >= seg_hi) j = t0;
        const int page = lds_pages[window_slot(j, shift, pg0)];
        const int64_t off = pool_row(page, p.hkv, w.g, shift, j & pmask, D) + c * 8;
        lds_dma16(kpool + off, &lds_ring[TG::ring_dst(stage, 0, wave, i)]);
        lds_dma16(vpool + off, &lds_ring[TG::ring_dst(stage, 1, wave, i)]);
      }
    };

    // Wait for tile t, then reuse the stage freed by the previous iteration
    // for tile t + AHEAD.
    auto advance = [&](int t) {
      // Tile t's loads are done once at most (tiles issued after it) * LPT are in flight.
      const int after = min(AHEAD - 1, nt - 1 - t);
      if (after >= 2) wait_vmcnt<2 * LPT>();
      else if (after == 1) wait_vmcnt<LPT>();
      else wait_vmcnt<0>();
      __syncthreads();  // all threads' loads of tile t landed; the freed stage is unused
      if (t + AHEAD < nt) issue(t + AHEAD, (t + AHEAD) % NST);
    };

#pragma unroll
    for (int st = 0; st < AHEAD; ++st)
      if (st < nt) issue(st, st);

    V8 pb[NS2][MB];
    for (int t = 0; t < ntp; ++t) {
      advance(t);
      if (!wave_active) continue;
      const int t0 = seg_lo + t * KT;
      f32x4 sacc[NKB][MB];
      // Rotated loop: the wave issues its matrix instructions at raised
      // priority, so that of the two waves sharing a SIMD the one with
      // matrix work to issue goes first while the other runs its softmax
      // (measured: wide beam 1.5%, the head_dim 64 4B layer 2-3% and the
      // cached-prefix prefill's cache segment 4% faster; the unrotated loop,
      // whose softmax sits between its two products, gains nothing).
      if (ROT) __builtin_amdgcn_s_setprio(1);
      s_tile(lds_kv[t % NST][0], sacc);
      if (ROT && t > 0) o_tile(lds_kv[(t - 1) % NST][1], pb);
      if (ROT) __builtin_amdgcn_s_setprio(0);
      softmax_tile(sacc, (t0 + KT <= w.k_hi) && (is_pre || causal1 ? t0 + KT - 1 <= c_first : !p.causal),
                   [&](int qb, int kk) { return (t0 + kk < w.k_hi) & (t0 + kk <= climit[qb]); }, pb);
      if (!ROT) o_tile(lds_kv[t % NST][1], pb);
    }
    if (ROT && wave_active && ntp > 0) o_tile(lds_kv[(ntp - 1) % NST][1], pb);
  }

  // ---- a split request: this workgroup leaves its chunk's partial state in
  // its slot and counts its arrival on the request's counter (per KV head and
  // query tile). The last to arrive merges all chunks' states (the exact
  // log-sum-exp rule, in chunk order) and finishes the request; the others are
  // done. No workgroup waits for another. The states and the counter are
  // accessed only with agent-coherent loads, stores and one atomic add, and a
  // state is counted only after its stores have completed, so no cache-wide
  // write-back or invalidation is needed. The last arrival also resets the
  // counter for the next launch.
  if (split) {
    const int64_t per = (int64_t)f.part_floats * 256;
    const int64_t nsub = (int64_t)p.hkv * p.n_qtiles;
    const int64_t sub = (int64_t)w.g * p.n_qtiles + w.qt;
    auto state = [&](int k) { return f.split_part + ((int64_t)(slot + k) * nsub + sub) * per; };
    auto put = [](float* q, float v) {
      __hip_atomic_store(q, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    auto get = [](const float* q) {
      return __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    {
      float* st = state(part);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int qb = 0; qb < MB; ++qb)
#pragma unroll
          for (int e = 0; e < 4; ++e) put(st + ((db * MB + qb) * 4 + e) * 256 + tid, oacc[db][qb][e]);
#pragma unroll
      for (int qb = 0; qb < MB; ++qb) {
        put(st + (NDB * MB * 4 + qb) * 256 + tid, mrow[qb]);
        put(st + (NDB * MB * 4 + MB + qb) * 256 + tid, lrow[qb]);
      }
    }
    // this thread's stores are complete (the clobber keeps them above it)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // and so are every other thread's; lds_pages is no longer read
    if (tid == 0) {
      int32_t* ctr = f.split_count + ((int64_t)w.b * p.hkv + w.g) * p.n_qtiles + w.qt;
      const int arrived = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = arrived == parts - 1 ? 1 : 0;
      if (last) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      lds_pages[0] = last;
    }
    __syncthreads();  // the state loads below are issued after the count was taken
    if (lds_pages[0] == 0) return;
    // The states are merged in chunk order, this workgroup's own read back like
    // the others, so the result does not depend on which chunk arrived last.
    for (int k = 0; k < parts; ++k) {
      const float* st = state(k);
      if (k == 0) {
#pragma unroll
        for (int qb = 0; qb < MB; ++qb) {
          mrow[qb] = get(st + (NDB * MB * 4 + qb) * 256 + tid);
          lrow[qb] = get(st + (NDB * MB * 4 + MB + qb) * 256 + tid);
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int e = 0; e < 4; ++e) oacc[db][qb][e] = get(st + ((db * MB + qb) * 4 + e) * 256 + tid);
        }
        continue;
      }
#pragma unroll
      for (int qb = 0; qb < MB; ++qb) {
        const float m2 = get(st + (NDB * MB * 4 + qb) * 256 + tid);
        const float l2 = get(st + (NDB * MB * 4 + MB + qb) * 256 + tid);
        const float m_new = fmaxf(mrow[qb], m2);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float a1 = fast_exp2((mrow[qb] - m_use) * c2);
        const float a2 = fast_exp2((m2 - m_use) * c2);
        mrow[qb] = m_new;
        lrow[qb] = lrow[qb] * a1 + l2 * a2;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            oacc[db][qb][e] = oacc[db][qb][e] * a1 + get(st + ((db * MB + qb) * 4 + e) * 256 + tid) * a2;
      }
    }
  }

  if constexpr (TAILS1) {  // the slot table, now that the prompt is done
    if (split) {
      sl_build(0);
    } else if constexpr (DEFER) {
      sl_commit(0, t_src, t_page);
      sl_build(256 * TR);
    }
  }

  // ---- MODE 1: each wave attends its own beams' tails (slot-table rows
  // u = (beam - kb_first) * n_tail + t) in 16-key sub-tiles, double-buffered
  // in its quarter of the now idle tile ring, with no workgroup barrier. A
  // tail key is visible only to its own beam's query rows.
  if constexpr (TAILS1) {
    __syncthreads();  // every wave is done with the ring; the slot table is visible
    if (f.dump_slots != nullptr) {  // debug: the table itself instead of the tails and output
      for (int u = tid; u < n_sl; u += 256)
        f.dump_slots[(((int64_t)w.b * p.hkv + w.g) * p.W + kb_first + u / ri.tail) * f.dump_pad +
                     u % ri.tail] = lds_tail[u];
      return;
    }
    if (n_tail > 0 && wave_active) {
      constexpr int KW = TG::KW;                                   // keys per sub-tile
      constexpr int NIW = TG::NIW;                                 // 1 KB loads each (K, and V)
      constexpr int NBUF = TG::NBUF;
      static_assert(TG::REGION >= 2 * TG::SUB && NIW >= 1 && TG::RING * (int)sizeof(T) == (int)sizeof(lds_kv),
                    "sub-tile must fit a wave's share of the ring");
      const int r_last = row_end - 1;
      const int u_lo = (row0 / p.group - kb_first) * n_tail;
      const int u_hi = (r_last / p.group - kb_first + 1) * n_tail;
      const int n_sub = (u_hi - u_lo + KW - 1) / KW;
      int tail_lo[MB];  // this lane's rows of the slot table: [tail_lo, tail_lo + n_tail)
#pragma unroll
      for (int qb = 0; qb < MB; ++qb) {
        const int r = row0 + qb * 16 + l16;
        tail_lo[qb] = r < row_end ? (r / p.group - kb_first) * n_tail : INT_MIN / 2;
      }
      // a finite row for sub-tile rows that carry no key (padding, invalid slots)
      const int64_t pad_row = ((int64_t)w.b * p.W + kb_first) * f.new_stride + (int64_t)w.g * D;
      auto issue_sub = [&](int sidx, int buf) {
#pragma unroll
        for (int i = 0; i < NIW; ++i) {
          const int r = TG::sub_row(i, lane);
          const int c = TG::sub_chunk(i, lane);
          const int u = u_lo + sidx * KW + r;
          const int32_t e = u < u_hi ? lds_tail[u] : -1;
          const T* ksrc;
          const T* vsrc;
          if (e >= 0) {
            ksrc = kpool + (int64_t)e * D + c * 8;
            vsrc = vpool + (int64_t)e * D + c * 8;
          } else {
            const int64_t o = e <= -2 ? ((int64_t)w.b * p.W + (-2 - e)) * f.new_stride + (int64_t)w.g * D
                                      : pad_row;
            ksrc = static_cast<const T*>(f.k_new) + o + c * 8;
            vsrc = static_cast<const T*>(f.v_new) + o + c * 8;
          }
          lds_dma16(ksrc, &lds_ring[TG::region_dst(wave, buf, 0, i)]);
          lds_dma16(vsrc, &lds_ring[TG::region_dst(wave, buf, 1, i)]);
        }
      };
      issue_sub(0, 0);
      if (NBUF == 2 && n_sub > 1) issue_sub(1, 1);
      for (int sidx = 0; sidx < n_sub; ++sidx) {
        const int buf = NBUF == 2 ? (sidx & 1) : 0;
        if (NBUF == 2 && sidx + 1 < n_sub) wait_vmcnt<2 * NIW>();
        else wait_vmcnt<0>();
        const T* lk = &lds_ring[TG::region_dst(wave, buf, 0, 0)];
        const T* lv = &lds_ring[TG::region_dst(wave, buf, 1, 0)];
        const int u0 = u_lo + sidx * KW;
        // ---- S^T = K Q^T for the query blocks whose beams own keys here
        f32x4 sacc[MB];
        bool act[MB];
#pragma unroll
        for (int qb = 0; qb < MB; ++qb) {
          const int r_lo = row0 + qb * 16;
          const int lo = (r_lo / p.group - kb_first) * n_tail;
          const int hi = ((min(r_lo + 16, row_end) - 1) / p.group - kb_first + 1) * n_tail;
          act[qb] = r_lo < row_end && lo < min(u0 + KW, u_hi) && hi > u0;
          sacc[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // With one query block per wave every operand read is issued before
        // the first is used: the K rows here, the V^T columns right after S^T
        // so that they land during the softmax (one LDS round trip per
        // sub-tile instead of one per operand; measured: the n-sample step,
        // whose tails are long, ~1% faster; at more blocks per wave the
        // registers cost more than the overlap gains).
        constexpr bool TPF = MB == 1;
        auto k_op = [&](int ds) { return *reinterpret_cast<const V8*>(&lk[TG::k_read(l16, ds * 4 + l4)]); };
        const int ra = 4 * l4 + (l16 >> 2);
        auto v_op = [&](int db) {
          return __builtin_bit_cast(u32x2, lds_read_tr(&lv[TG::v_read(ra, db * 16 + 4 * (l16 & 3))]));
        };
        V8 ka[TPF ? NDS : 1];
        if constexpr (TPF) {
#pragma unroll
          for (int ds = 0; ds < NDS; ++ds) ka[ds] = k_op(ds);
        }
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
          const V8 a = TPF ? ka[TPF ? ds : 0] : k_op(ds);
#pragma unroll
          for (int qb = 0; qb < MB; ++qb)
            if (act[qb]) sacc[qb] = Mfma<T>::mma(a, qv[qb][ds], sacc[qb]);
        }
        u32x2 va[TPF ? NDB : 1];
        if constexpr (TPF) {
#pragma unroll
          for (int db = 0; db < NDB; ++db) va[db] = v_op(db);
        }
        // ---- mask (own beam, valid slot) and online softmax
        u32x2 pb[MB];
#pragma unroll
        for (int qb = 0; qb < MB; ++qb) {
          if (!act[qb]) continue;
          float mx = -INFINITY;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int u = u0 + l4 * 4 + e;
            const bool vis = u >= tail_lo[qb] && u < tail_lo[qb] + n_tail && lds_tail[u] != -1;
            const float sv = vis ? sacc[qb][e] : -INFINITY;
            sacc[qb][e] = sv;
            mx = fmaxf(mx, sv);
          }
          // the same lane-wise test as the prompt loop's
          if (__builtin_expect(__builtin_amdgcn_ballot_w64(mx > mrow[qb] + lazy_keys) != 0, 0)) {
            asm volatile("" ::: "memory");
            mx = max4x16(mx);
            const float m_new = fmaxf(mrow[qb], mx);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = fast_exp2((mrow[qb] - m_use) * c2);
            mrow[qb] = m_new;
            lrow[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) oacc[db][qb] *= alpha;
          }
          const float moff = mrow[qb] == -INFINITY ? 0.f : -mrow[qb] * c2;
          T e4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pr = fast_exp2(fmaf(sacc[qb][e], c2, moff));
            lrow[qb] += pr;
            e4[e] = Traits<T>::from_f(pr);
          }
          pb[qb] = __builtin_bit_cast(u32x2, e4);
        }
        // ---- O^T += V^T P^T over the 16 keys (V^T operands by transpose reads)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const u32x2 a = TPF ? va[TPF ? db : 0] : v_op(db);
#pragma unroll
          for (int qb = 0; qb < MB; ++qb)
            if (act[qb]) oacc[db][qb] = Mfma<T>::mma16(a, pb[qb], oacc[db][qb]);
        }
        // refill this buffer once its LDS reads are done
        if (NBUF == 2 ? sidx + 2 < n_sub : sidx + 1 < n_sub) {
          wait_lgkmcnt0();
          issue_sub(NBUF == 2 ? sidx + 2 : sidx + 1, buf);
        }
      }
    }
  }

  // ---- MODE 2: each beam's tail joins the same online softmax, key by key
  if constexpr (MODE == 2) {
    if (n_tail > 0 && wave_active) {
      const int jcur = ri.seq - 1;
      constexpr int TC = 2;  // tail keys in flight together
#pragma unroll
      for (int qb = 0; qb < MB; ++qb) {
        const int r = row0 + qb * 16 + l16;
        const bool row_ok = r < row_end;
        const int kbeam = row_ok ? r / p.group : kb_first;
        const int h = w.g * p.group + (row_ok ? r % p.group : 0);
        // this lane's columns of O^T: d = db * 16 + 4 * l4 + i (query kept packed)
        u32x2 qraw[NDB];
        {
          const T* qr = static_cast<const T*>(p.q) + (((int64_t)w.b * p.W + kbeam) * p.hq + h) * D + 4 * l4;
#pragma unroll
          for (int db = 0; db < NDB; ++db) qraw[db] = *reinterpret_cast<const u32x2*>(qr + db * 16);
        }
        for (int t0 = 0; t0 < n_tail; t0 += TC) {
          const T* kr[TC];
          const T* vr[TC];
          bool ok[TC];
#pragma unroll
          for (int c = 0; c < TC; ++c) {
            const int t = t0 + c;
            int32_t e = -1;
            if (t < n_tail && row_ok)
              e = resolve_fused_slot(p, f, w.b, kbeam, w.g, ri.prefix + t, jcur);
            ok[c] = e != -1;
            if (e >= 0) {
              kr[c] = kpool + (int64_t)e * D + 4 * l4;
              vr[c] = vpool + (int64_t)e * D + 4 * l4;
            } else {  // the current token of beam -e-2 (or a skipped key: any valid row)
              const int src = e <= -2 ? -2 - e : 0;
              const int64_t o = ((int64_t)w.b * p.W + src) * f.new_stride + (int64_t)w.g * D + 4 * l4;
              kr[c] = static_cast<const T*>(f.k_new) + o;
              vr[c] = static_cast<const T*>(f.v_new) + o;
            }
          }
          // scores of the TC keys
          float pr[TC], alpha = 1.f;
          {
            u32x2 kraw[TC][NDB];
#pragma unroll
            for (int c = 0; c < TC; ++c)
#pragma unroll
              for (int db = 0; db < NDB; ++db) kraw[c][db] = *reinterpret_cast<const u32x2*>(kr[c] + db * 16);
            float sc[TC];
#pragma unroll
            for (int c = 0; c < TC; ++c) {
              float part = 0.f;
#pragma unroll
              for (int db = 0; db < NDB; ++db) {
                const T* ke = reinterpret_cast<const T*>(&kraw[c][db]);
                const T* qe = reinterpret_cast<const T*>(&qraw[db]);
#pragma unroll
                for (int i = 0; i < 4; ++i) part = fmaf(Traits<T>::to_f(qe[i]), Traits<T>::to_f(ke[i]), part);
              }
              part = sum4x16(part);
              sc[c] = ok[c] ? part : -INFINITY;
            }
            float mx = sc[0];
#pragma unroll
            for (int c = 1; c < TC; ++c) mx = fmaxf(mx, sc[c]);
            const float m_new = fmaxf(mrow[qb], mx);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            alpha = fast_exp2((mrow[qb] - m_use) * c2);
            float psum = 0.f;
#pragma unroll
            for (int c = 0; c < TC; ++c) {
              pr[c] = fast_exp2((sc[c] - m_use) * c2);
              psum += pr[c];
            }
            mrow[qb] = m_new;
            // lrow holds this lane's share of the row sum: add each key once
            lrow[qb] = fmaf(lrow[qb], alpha, l4 == 0 ? psum : 0.f);
          }
          // values of the TC keys
          {
            u32x2 vraw[TC][NDB];
#pragma unroll
            for (int c = 0; c < TC; ++c)
#pragma unroll
              for (int db = 0; db < NDB; ++db) vraw[c][db] = *reinterpret_cast<const u32x2*>(vr[c] + db * 16);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                float acc = oacc[db][qb][i] * alpha;
#pragma unroll
                for (int c = 0; c < TC; ++c)
                  acc = fmaf(pr[c], Traits<T>::to_f(reinterpret_cast<const T*>(&vraw[c][db])[i]), acc);
                oacc[db][qb][i] = acc;
              }
            }
          }
        }
      }
    }
  }

  // ---- epilogue: normalise and write the partial state (or the final output)
  [[maybe_unused]] const __amdgpu_buffer_rsrc_t o_rsrc =
      raw_rsrc(p.o_part, (uint32_t)((int64_t)p.n_split * p.rows_total * p.hq * D * 4));
  [[maybe_unused]] const __amdgpu_buffer_rsrc_t l_rsrc =
      raw_rsrc(p.lse_part, (uint32_t)((int64_t)p.n_split * p.rows_total * p.hq * 4));
#pragma unroll
  for (int qb = 0; qb < MB; ++qb) {
    const float lt = sum4x16(lrow[qb]);
    const int r = row0 + qb * 16 + l16;
    if (!wave_active || r >= row_end) continue;
    const int hh = r % p.group;
    const int t = r / p.group;
    const int64_t grow = is_pre ? (int64_t)ri.q_off + t
                                 : ((int64_t)w.b * p.W + t / p.q_len) * p.q_len + t % p.q_len;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse = lt > 0.f ? mrow[qb] * p.scale + __logf(lt) : -INFINITY;
    if constexpr (FUSED || PREFILL) {
      const int64_t ohead = grow * p.hq + w.g * p.group + hh;
      T* orow = static_cast<T*>(f.o_out) + ohead * D;
      if constexpr (MB <= 2) {
        // Lane row l4 holds columns 4*l4..4*l4+3 of each 16-column block. One
        // permlane16 swap per dword pairs blocks db and db+1 across neighbouring
        // lane rows, so even rows hold 8 columns of block db and odd rows 8 of
        // block db+1: 16 bytes per lane and 64 contiguous bytes per row and
        // store, whole memory segments for the streaming stores. (At three
        // blocks per wave the swaps cost registers the loop does not have.)
        static_assert(NDB % 2 == 0, "output blocks are stored in pairs");
        T* op = orow + (l4 & 1) * 16 + (l4 >> 1) * 8;
#pragma unroll
        for (int db = 0; db < NDB; db += 2) {
          T a4[4], b4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a4[e] = Traits<T>::from_f(oacc[db][qb][e] * inv);
            b4[e] = Traits<T>::from_f(oacc[db + 1][qb][e] * inv);
          }
          const u32x2 au = __builtin_bit_cast(u32x2, a4);
          const u32x2 bu = __builtin_bit_cast(u32x2, b4);
          const unsigned a0 = au[0], a1 = au[1], b0 = bu[0], b1 = bu[1];
          const auto s0 = __builtin_amdgcn_permlane16_swap(a0, b0, false, false);
          const auto s1 = __builtin_amdgcn_permlane16_swap(a1, b1, false, false);
          const unsigned x0 = s0[0], y0 = s0[1], x1 = s1[0], y1 = s1[1];
          const u32x4 v = {x0, x1, y0, y1};
          store_maybe_stream(reinterpret_cast<u32x4*>(op + db * 16), v, fused && f.stream_out);
        }
      } else {
        T* op = orow + l4 * 4;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          T e4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) e4[e] = Traits<T>::from_f(oacc[db][qb][e] * inv);
          *reinterpret_cast<u32x2*>(op + db * 16) = __builtin_bit_cast(u32x2, e4);
        }
      }
      if (l4 == 0 && f.lse_out != nullptr) {
        if constexpr (MB <= 2) store_maybe_stream(f.lse_out + ohead, lse, fused && f.stream_out);
        else f.lse_out[ohead] = lse;
      }
    } else if constexpr (MODE == 5) {
      // read back by the last chunk to finish, maybe on another XCD: agent-coherent
      // (sc1) stores, 16 bytes each; offsets fit 32 bits (checked by the host)
      const int64_t ohead = ((int64_t)w.split * p.rows_total + grow) * p.hq + w.g * p.group + hh;
      const uint32_t ob = (uint32_t)((ohead * D + l4 * 4) * 4);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4, oacc[db][qb] * inv), o_rsrc, ob + db * 64, 0, kCoherentAgent);
      if (l4 == 0)
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lse), l_rsrc,
                                              (uint32_t)(ohead * 4), 0, kCoherentAgent);
    } else {
      const int64_t ohead = ((int64_t)w.split * p.rows_total + grow) * p.hq + w.g * p.group + hh;
      float* op = p.o_part + ohead * D + l4 * 4;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        *reinterpret_cast<f32x4*>(op + db * 16) = oacc[db][qb] * inv;
      if (l4 == 0) p.lse_part[ohead] = lse;
    }
  }

  // ---- MODE 5, the one-launch cached-prefix decode: each cache chunk counts
  // its arrival per (request, KV head) once its partial state is stored; the
  // last to arrive merges all chunks' states, in chunk order, with this call's
  // row (its own key, read from k_new/v_new) into the output, and writes the
  // new row into its page. No workgroup waits for another.
  if constexpr (MODE == 5) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // every thread's partial-state stores are complete; the ring is idle
    if (tid == 0) {
      int32_t* ctr = f.split_count + (int64_t)w.b * p.hkv + w.g;
      const int arrived = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = arrived == p.n_split - 1 ? 1 : 0;
      if (last) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      lds_pages[0] = last;
    }
    __syncthreads();
    if (lds_pages[0] == 0) return;
    // The chunks' states were stored with agent-coherent stores, complete before
    // their counts; they are read back with agent-coherent (sc1) loads.
    //
    // Thread (slice, row, chunk of 4 columns) loads the lse and the 4 output
    // columns of its slice's chunks (every ns-th one), all in one round trip,
    // and folds them with its own running maximum; the ns slices are then
    // joined, with this call's new row, through LDS. A row's CH chunks are CH
    // adjacent lanes of one wave (CH divides 64), so the new row's score is a
    // lane reduction.
    constexpr int CH = D / 4;                 // 4-column chunks of a row
    const int np = p.group * CH;              // (row, chunk) pairs; the host checked np <= 256
    const int ns = 256 / np;                  // slices of threads
    const int pair = tid % np, slice = tid / np;
    const bool act = slice < ns;
    const int row = pair / CH, ch = pair % CH;
    const int h = w.g * p.group + row;
    const int64_t hs = (int64_t)p.rows_total * p.hq;  // entries of one chunk's lse
    const int64_t lrow = (int64_t)w.b * p.hq + h;
    const int64_t nrow = (int64_t)w.b * f.new_stride + (int64_t)w.g * D + ch * 4;
    const u32x2 q2 = *reinterpret_cast<const u32x2*>(static_cast<const T*>(p.q) + lrow * D + ch * 4);
    const u32x2 k2 = *reinterpret_cast<const u32x2*>(static_cast<const T*>(f.k_new) + nrow);
    const u32x2 v2 = *reinterpret_cast<const u32x2*>(static_cast<const T*>(f.v_new) + nrow);
    constexpr int NB = 32;  // chunks in flight per thread
    const uint32_t ob = (uint32_t)((lrow * D + ch * 4) * 4), lb = (uint32_t)(lrow * 4);
    const uint32_t ostep = (uint32_t)(hs * D * 4), lstep = (uint32_t)(hs * 4);
    f32x4 o[NB];
    float lv[NB];
    auto load_batch = [&](int sp0) {
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const uint32_t sp = (uint32_t)(sp0 + k * ns);
        const bool in = act && (int)sp < p.n_split;
        lv[k] = in ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                   l_rsrc, lb + sp * lstep, 0, kCoherentAgent))
                   : -INFINITY;
        o[k] = in ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  o_rsrc, ob + sp * ostep, 0, kCoherentAgent))
                  : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    };
    // running state of this thread's chunks: max m_s, weight sum den_s, weighted sum acc
    float m_s = -INFINITY, den_s = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto add_batch = [&]() {
      float bm = lv[0];
#pragma unroll
      for (int k = 1; k < NB; ++k) bm = fmaxf(bm, lv[k]);
      const float mn = fmaxf(m_s, bm);
      if (mn == -INFINITY) return;  // only empty chunks so far
      const float sc = fast_exp2((m_s - mn) * kLog2e);  // m_s = -inf: 0, and acc is 0
      acc *= sc;
      den_s *= sc;
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const float wt = fast_exp2((lv[k] - mn) * kLog2e);  // empty or absent chunk: 0
        if (wt > 0.f) {
          den_s += wt;
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = fmaf(wt, o[k][e], acc[e]);
        }
      }
      m_s = mn;
    };
    load_batch(slice);
    float s_new;  // the new row's score, natural-log units like the chunks' lse
    {
      const T* qe = reinterpret_cast<const T*>(&q2);
      const T* ke = reinterpret_cast<const T*>(&k2);
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) dot = fmaf(Traits<T>::to_f(qe[e]), Traits<T>::to_f(ke[e]), dot);
      dot = row16_sum(dot);
      if constexpr (CH >= 32) dot += xor16(dot);
      if constexpr (CH == 64) dot += xor32(dot);
      s_new = dot * p.scale;
    }
    add_batch();
    for (int sp0 = slice + NB * ns; sp0 < p.n_split; sp0 += NB * ns) {
      load_batch(sp0);
      add_batch();
    }
    // LDS (the idle ring): the states of slices 1..ns-1
    f32x4* sh_acc = reinterpret_cast<f32x4*>(lds_ring);
    float2* sh_md = reinterpret_cast<float2*>(sh_acc + 256);
    if (act && slice > 0) {
      sh_acc[(slice - 1) * np + pair] = acc;
      sh_md[(slice - 1) * np + pair] = float2{m_s, den_s};
    }
    __syncthreads();
    if (act && slice == 0) {
      float M = fmaxf(s_new, m_s);
      for (int sl = 1; sl < ns; ++sl) M = fmaxf(M, sh_md[(sl - 1) * np + pair].x);
      float c = fast_exp2((m_s - M) * kLog2e);
      acc *= c;
      float den = den_s * c;
      for (int sl = 1; sl < ns; ++sl) {
        const float2 md = sh_md[(sl - 1) * np + pair];
        c = fast_exp2((md.x - M) * kLog2e);
        acc += sh_acc[(sl - 1) * np + pair] * c;
        den = fmaf(md.y, c, den);
      }
      const float w_new = fast_exp2((s_new - M) * kLog2e);
      den += w_new;
      const T* ve = reinterpret_cast<const T*>(&v2);
      const float inv = 1.f / den;
      T e4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) e4[e] = Traits<T>::from_f(fmaf(w_new, Traits<T>::to_f(ve[e]), acc[e]) * inv);
      *reinterpret_cast<u32x2*>(static_cast<T*>(f.o_out) + lrow * D + ch * 4) = __builtin_bit_cast(u32x2, e4);
      if (ch == 0 && f.lse_out != nullptr) f.lse_out[lrow] = M + __logf(den);
    }
    // this call's row into its page (KV head g's slice)
    if (tid < CPR) {
      const int32_t slot = f.new_slots[w.b];
      if (slot < 0 || (int64_t)slot >= ((int64_t)p.num_pages << shift)) {
        if (tid == 0)
          record_fault(&p.hdr->error_bits, &p.hdr->fault_count, &p.hdr->first_value,
                       kErrWriteSlot, slot);
      } else {
        const int64_t src = (int64_t)w.b * f.new_stride + (int64_t)w.g * D + tid * 8;
        const int64_t dst = pool_row(slot >> shift, p.hkv, w.g, shift, slot & pmask, D) + tid * 8;
        *reinterpret_cast<u32x4*>(static_cast<T*>(f.k_pool_w) + dst) =
            *reinterpret_cast<const u32x4*>(static_cast<const T*>(f.k_new) + src);
        *reinterpret_cast<u32x4*>(static_cast<T*>(f.v_pool_w) + dst) =
            *reinterpret_cast<const u32x4*>(static_cast<const T*>(f.v_new) + src);
      }
    }
  }

  // ---- the current tokens (see above): the stores of the rows loaded in the
  // prologue, or loads and stores here (the unrolled batch holds all of a wide
  // beam's tasks)
  if (TW_EARLY && tw_early) {
    tw_store(0, e_page, e_kd, e_vd);
  } else if (n_tw > 0) {
    constexpr int TW = 16;
    for (int base = 0; base < n_tw; base += 256 * TW) {
      int32_t page[TW];
      u32x4 kd[TW], vd[TW];
      tw_load(base, page, kd, vd);
      tw_store(base, page, kd, vd);
    }
  }
}

template <typename T, int D, int MB, int KT, int NST, int MODE>
__global__ __launch_bounds__(256, (prefix_min_blocks<D, MB>())) void prefix_mfma_kernel(PrefixParams p,
                                                                                          FusedParams f) {
  prefix_body<T, D, MB, KT, NST, MODE>(p, f, blockIdx.x, false);
}

// A mixed step in one launch: n_dec beam-step workgroups (dp, df) and n_pre
// context workgroups (pp, pf). Chunks of 256 of each alternate while both
// last, so that the first round puts a beam-step workgroup (bandwidth-bound)
// and a context workgroup (latency- and matrix-bound) side by side on a CU
// rather than one kind after the other.
template <typename T, int D, int KT, int NST>
__global__ __launch_bounds__(256, (prefix_min_blocks<D, 1>())) void mixed_step_kernel(
    PrefixParams dp, FusedParams df, PrefixParams pp, FusedParams pf, int n_dec, int n_pre) {
  constexpr int C = 256;
  int rem = blockIdx.x, done_d = 0, done_p = 0;
  bool pre = false;
  int idx = 0;
  for (int c = 0;; ++c) {  // at most (n_dec + n_pre) / 256 + 2 chunks; rem < n_dec + n_pre
    const bool dec_turn = done_d < n_dec && ((c & 1) == 0 || done_p >= n_pre);
    const int cnt = dec_turn ? min(C, n_dec - done_d) : min(C, n_pre - done_p);
    if (rem < cnt) {
      pre = !dec_turn;
      idx = (dec_turn ? done_d : done_p) + rem;
      break;
    }
    rem -= cnt;
    if (dec_turn) done_d += cnt;
    else done_p += cnt;
  }
  // one copy of the body; the parameters are picked per workgroup
  prefix_body<T, D, 1, KT, NST, 4>(pre ? pp : dp, pre ? pf : df, idx, pre);
}

// Two plans' shared-key attention in one launch (MODE 0, one 16-row query
// block per wave): the first n_a workgroups are plan a's work items, the rest
// plan b's; each writes its own plan's partial states. For two small segments
// of one call (the cached rows and this call's rows) one launch instead of two.
template <typename T, int D, int KT, int NST>
__global__ __launch_bounds__(256, (prefix_min_blocks<D, 1>())) void prefix_two_kernel(
    PrefixParams a, PrefixParams b, int n_a) {
  const FusedParams none{};
  const bool second = (int)blockIdx.x >= n_a;
  prefix_body<T, D, 1, KT, NST, 0>(second ? b : a, none,
                                          second ? (int)blockIdx.x - n_a : (int)blockIdx.x, false);
}

// f32: one wave per query row, lanes split head_dim, keys in chunks of 8.
template <int D>
__global__ __launch_bounds__(256) void prefix_simt_kernel(PrefixParams p) {
  constexpr int EPL = D / 64;
  constexpr int CHUNK = 8;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int bid = blockIdx.x;
  const int qt = bid % p.n_qtiles;
  bid /= p.n_qtiles;
  const int split = bid % p.n_split;
  bid /= p.n_split;
  const int g = bid % p.hkv;
  const int b = bid / p.hkv;
  const ReqInfo ri = p.req[b];
  const int M = p.W * p.q_len * p.group;
  const int r = qt * 4 + wave;
  if (r >= M) return;
  int k_lo = p.split_keys > 0 ? split * p.split_keys : 0;
  int k_hi = p.split_keys > 0 ? min(ri.valid, k_lo + p.split_keys) : ri.valid;
  const int hh = r % p.group;
  const int t = r / p.group;
  const int i = t % p.q_len;
  const int kbeam = t / p.q_len;
  if (p.causal) k_hi = min(k_hi, ri.n_keys - p.q_len + i + 1);
  const int ps = 1 << p.page_shift;
  const int64_t grow = ((int64_t)b * p.W + kbeam) * p.q_len + i;
  const int h = g * p.group + hh;
  const float* qp = static_cast<const float*>(p.q) + (grow * p.hq + h) * D + lane * EPL;
  const float* kpool = static_cast<const float*>(p.k_pool);
  const float* vpool = static_cast<const float*>(p.v_pool);
  float q[EPL], acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    q[e] = qp[e];
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int j0 = k_lo; j0 < k_hi; j0 += CHUNK) {
    float kr[CHUNK][EPL], vr[CHUNK][EPL];
    bool ok[CHUNK];
#pragma unroll
    for (int c = 0; c < CHUNK; ++c) {
      const int j = j0 + c;
      ok[c] = false;
      if (j < k_hi) {
        const int32_t page = p.pages[ri.page_off + (j >> p.page_shift)];
        if (page >= 0 && page < p.num_pages) {
          ok[c] = true;
          const int64_t off = (((int64_t)page * p.hkv + g) * ps + (j & (ps - 1))) * D + lane * EPL;
#pragma unroll
          for (int e = 0; e < EPL; ++e) {
            kr[c][e] = kpool[off + e];
            vr[c][e] = vpool[off + e];
          }
        } else if (lane == 0) {
          record_fault(&p.hdr->error_bits, &p.hdr->fault_count, &p.hdr->first_value,
                       kErrPrefixPage, page);
        }
      }
      if (!ok[c]) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) kr[c][e] = vr[c][e] = 0.f;
      }
    }
    float s[CHUNK], cmax = -INFINITY;
#pragma unroll
    for (int c = 0; c < CHUNK; ++c) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) part = fmaf(q[e], kr[c][e], part);
      s[c] = ok[c] ? wave_sum(part) * p.scale_log2e : -INFINITY;
      cmax = fmaxf(cmax, s[c]);
    }
    const float m_new = fmaxf(m, cmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
#pragma unroll
    for (int c = 0; c < CHUNK; ++c) {
      const float pc = fast_exp2(s[c] - m_use);
      l += pc;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(pc, vr[c][e], acc[e]);
    }
    m = m_new;
  }
  const int64_t ohead = ((int64_t)split * p.rows_total + grow) * p.hq + h;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) p.o_part[ohead * D + lane * EPL + e] = acc[e] * inv;
  if (lane == 0) p.lse_part[ohead] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
}

// Tile size and pipeline depth per head_dim: 64 KB of K/V stages per workgroup.
template <typename T, int MODE>
static void launch_mfma(const PrefixParams& p, const FusedParams& f, int head_dim, int mb,
                        unsigned blocks, hipStream_t s) {
#define BSP_PFX(DD, MBB, KTT, NS) \
  prefix_mfma_kernel<T, DD, MBB, KTT, NS, MODE><<<blocks, 256, 0, s>>>(p, f)
  if (head_dim == 64) {
    if (mb == 1) BSP_PFX(64, 1, 64, 4);
    else if (mb == 2) BSP_PFX(64, 2, 64, 4);
    else BSP_PFX(64, 3, 64, 4);
  } else if (head_dim == 128) {
    // The fused step at one or two query blocks per wave, and the partial-state
    // kernel at one, stream 64-key tiles through a two-stage ring (the same LDS
    // as four stages of 32 keys, half the barriers, waits and row-max
    // reductions per key): 3-4% faster at one block (fused), ~1-2% at two and
    // ~2.5% for the partial-state kernel. At three blocks the 64-key tile
    // spills registers.
    if (mb == 1) {
      if constexpr (MODE == 1 || MODE == 0) BSP_PFX(128, 1, 64, 2);
      else BSP_PFX(128, 1, 32, 4);
    } else if (mb == 2) {
      if constexpr (MODE == 1) BSP_PFX(128, 2, 64, 2);
      else BSP_PFX(128, 2, 32, 4);
    } else {
      BSP_PFX(128, 3, 32, 4);
    }
  } else {  // pick_mb: one query block per wave at head_dim 256
    BSP_PFX(256, 1, 32, 2);
  }
#undef BSP_PFX
}

hipError_t launch_prefix(const PrefixParams& p, int dtype, int head_dim, int rows_per_tile,
                         hipStream_t s) {
  const unsigned blocks = (unsigned)(p.B * p.hkv * p.n_split * p.n_qtiles);
  if (blocks == 0) return hipSuccess;
  if (dtype == BSP_F32) {
    if (head_dim == 64) prefix_simt_kernel<64><<<blocks, 256, 0, s>>>(p);
    else if (head_dim == 128) prefix_simt_kernel<128><<<blocks, 256, 0, s>>>(p);
    else prefix_simt_kernel<256><<<blocks, 256, 0, s>>>(p);
  } else {
    const int mb = rows_per_tile / 64;
    if (mb < 1 || mb > pick_mb(head_dim, 64 * 3) || rows_per_tile % 64 != 0)
      return hipErrorInvalidValue;
    const FusedParams none{};
    if (dtype == BSP_F16) launch_mfma<_Float16, 0>(p, none, head_dim, mb, blocks, s);
    else launch_mfma<__bf16, 0>(p, none, head_dim, mb, blocks, s);
  }
  return hipGetLastError();
}

bool cached_decode_supported(int group, int head_dim) {
  // the merge's (row, chunk of 4 columns) pairs fit the 256 threads
  return group * head_dim / 4 <= 256;
}

hipError_t launch_cached_decode(const PrefixParams& p, const FusedParams& f, int dtype,
                                int head_dim, hipStream_t s) {
  const unsigned blocks = (unsigned)(p.B * p.hkv * p.n_split * p.n_qtiles);
  if (blocks == 0) return hipSuccess;
  if (dtype != BSP_F16 && dtype != BSP_BF16) return hipErrorInvalidValue;
  if (!cached_decode_supported(p.group, head_dim)) return hipErrorInvalidValue;
#define BSP_CD(TT, DD, KTT, NS) prefix_mfma_kernel<TT, DD, 1, KTT, NS, 5><<<blocks, 256, 0, s>>>(p, f)
  if (dtype == BSP_F16) {
    if (head_dim == 64) BSP_CD(_Float16, 64, 64, 4);
    else if (head_dim == 128) BSP_CD(_Float16, 128, 64, 2);
    else BSP_CD(_Float16, 256, 32, 2);
  } else {
    if (head_dim == 64) BSP_CD(__bf16, 64, 64, 4);
    else if (head_dim == 128) BSP_CD(__bf16, 128, 64, 2);
    else BSP_CD(__bf16, 256, 32, 2);
  }
#undef BSP_CD
  return hipGetLastError();
}

hipError_t launch_prefix_two(const PrefixParams& a, const PrefixParams& b, int dtype, int head_dim,
                             hipStream_t s) {
  const int n_a = a.B * a.hkv * a.n_split * a.n_qtiles;
  const int n_b = b.B * b.hkv * b.n_split * b.n_qtiles;
  const unsigned blocks = (unsigned)(n_a + n_b);
  if (blocks == 0) return hipSuccess;
  if (dtype != BSP_F16 && dtype != BSP_BF16) return hipErrorInvalidValue;
#define BSP_TWO(TT, DD, KTT, NS) prefix_two_kernel<TT, DD, KTT, NS><<<blocks, 256, 0, s>>>(a, b, n_a)
  if (dtype == BSP_F16) {
    if (head_dim == 64) BSP_TWO(_Float16, 64, 64, 4);
    else if (head_dim == 128) BSP_TWO(_Float16, 128, 64, 2);
    else BSP_TWO(_Float16, 256, 32, 2);
  } else {
    if (head_dim == 64) BSP_TWO(__bf16, 64, 64, 4);
    else if (head_dim == 128) BSP_TWO(__bf16, 128, 64, 2);
    else BSP_TWO(__bf16, 256, 32, 2);
  }
#undef BSP_TWO
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefixParams& p, const FusedParams& f, int dtype, int head_dim,
                          int mb, int n_items, hipStream_t s) {
  const unsigned blocks = (unsigned)(n_items * p.hkv);
  if (blocks == 0) return hipSuccess;
// 64-key tiles in two stages at head_dim 128 and one or two query blocks per
// wave (as in the fused step: ~5% faster on short chunks), else four stages.
#define BSP_PRE(TT, DD, MBB, KTT)                                                   \
  prefix_mfma_kernel<TT, DD, MBB, KTT,                                             \
                     (KTT == 64 && DD == 128) || (DD == 256 && MBB == 1) ? 2 : 4, \
                     3><<<blocks, 256, 0, s>>>(p, f)
#define BSP_PRE_T(TT)                                      \
  if (head_dim == 64) {                                    \
    if (mb == 1) BSP_PRE(TT, 64, 1, 64);                   \
    else if (mb == 2) BSP_PRE(TT, 64, 2, 64);              \
    else BSP_PRE(TT, 64, 3, 64);                           \
  } else if (head_dim == 128) {                            \
    if (mb == 1) BSP_PRE(TT, 128, 1, 64);                  \
    else if (mb == 2) BSP_PRE(TT, 128, 2, 64);             \
    else BSP_PRE(TT, 128, 3, 32);                          \
  } else {                                                 \
    if (mb == 1) BSP_PRE(TT, 256, 1, 32);                  \
    else BSP_PRE(TT, 256, 2, 32);                          \
  }
  static_assert(prefill_max_mb(64) == 3 && prefill_max_mb(128) == 3 && prefill_max_mb(256) == 2,
                "instantiated tiles");
  if (dtype == BSP_F16) {
    BSP_PRE_T(_Float16)
  } else {
    BSP_PRE_T(__bf16)
  }
#undef BSP_PRE_T
#undef BSP_PRE
  return hipGetLastError();
}

bool mixed_step_supported(const PrefixParams& dp, const FusedParams& df, int dtype, int head_dim,
                          int rows_per_req, int tail_pad, int pre_mb) {
  if (dtype == BSP_F32 || head_dim > 128 || pre_mb != 1) return false;
  if (pick_mb(head_dim, rows_per_req) != 1 || dp.n_qtiles != 1) return false;
  if (df.split_count != nullptr) return false;
  const int nbt_max = min(dp.W, 63 / dp.group + 2);
  return (int64_t)nbt_max * tail_pad <= kTailSlots;  // the beam step's tails in the LDS table
}

hipError_t launch_mixed_step(const PrefixParams& dp, const FusedParams& df, const PrefixParams& pp,
                             const FusedParams& pf, int dtype, int head_dim, int n_pre_items,
                             hipStream_t s) {
  const int n_dec = dp.B * dp.hkv * dp.n_qtiles;
  const int n_pre = n_pre_items * pp.hkv;
  const unsigned blocks = (unsigned)(n_dec + n_pre);
  if (blocks == 0) return hipSuccess;
#define BSP_MIX(TT, DD, KTT, NS) \
  mixed_step_kernel<TT, DD, KTT, NS><<<blocks, 256, 0, s>>>(dp, df, pp, pf, n_dec, n_pre)
  if (dtype == BSP_F16) {  // head_dim 64 or 128 (mixed_step_supported)
    if (head_dim == 64) BSP_MIX(_Float16, 64, 64, 4);
    else BSP_MIX(_Float16, 128, 64, 2);
  } else {
    if (head_dim == 64) BSP_MIX(__bf16, 64, 64, 4);
    else BSP_MIX(__bf16, 128, 64, 2);
  }
#undef BSP_MIX
  return hipGetLastError();
}

bool decode_uses_slot_table(int head_dim, int rows_per_req, int W, int group, int tail_pad) {
  // beams with a row in one query tile, at most; their tail slots must fit the LDS table
  const int nbt_max = min(W, (64 * pick_mb(head_dim, rows_per_req) - 1) / group + 2);
  return (int64_t)nbt_max * tail_pad <= kTailSlots;
}

hipError_t launch_decode_step(const PrefixParams& p, const FusedParams& f, int dtype,
                              int head_dim, int rows_per_req, int n_items, int tail_pad,
                              hipStream_t s) {
  const unsigned blocks = (unsigned)(n_items * p.hkv * p.n_qtiles);
  if (blocks == 0) return hipSuccess;
  const int mb = pick_mb(head_dim, rows_per_req);
  if (decode_uses_slot_table(head_dim, rows_per_req, p.W, p.group, tail_pad)) {
    if (dtype == BSP_F16) launch_mfma<_Float16, 1>(p, f, head_dim, mb, blocks, s);
    else launch_mfma<__bf16, 1>(p, f, head_dim, mb, blocks, s);
  } else {
    if (dtype == BSP_F16) launch_mfma<_Float16, 2>(p, f, head_dim, mb, blocks, s);
    else launch_mfma<__bf16, 2>(p, f, head_dim, mb, blocks, s);
  }
  return hipGetLastError();
}

}  // namespace bsp
