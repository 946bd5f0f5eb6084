// CPU model of the shared-key kernel's addressing (prefix_attn.hip): it drives
// the kernel's loops (work items, page windows, key tiles, waves, lanes, tail
// sub-tiles, operand reads, token writes) through the same offset functions the
// kernel uses (tile_index.h) and checks every LDS offset against its array and
// every global offset against its buffer, for every instantiation the
// launchers use and for the beam, cached-prefix and prefill shapes of the
// tests and the bench. Exit status 0 when everything is in range; each
// violation is printed.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "../../beam_search_shared_amd/csrc/tile_index.h"

namespace {

constexpr int kPageWin = 1024;     // page ids per LDS window (prefix_attn.hip)
constexpr int kTailSlots = 3072;   // LDS tail-slot table entries (prefix_attn.hip)
constexpr int kLdsPerCu = 160 * 1024;

long g_checks = 0, g_bad = 0;

void need(bool ok, const std::string& what) {
  ++g_checks;
  if (!ok) {
    if (g_bad < 40) std::printf("OUT OF RANGE: %s\n", what.c_str());
    ++g_bad;
  }
}

struct Shape {
  const char* name;
  int hkv, group, W, ps;
  std::vector<int> P, T;  // prompt (shared keys) and tail length per request
};

uint64_t g_rng = 88172645463325252ull;
int draw(int lo, int hi) {  // inclusive
  g_rng ^= g_rng << 13;
  g_rng ^= g_rng >> 7;
  g_rng ^= g_rng << 17;
  return lo + (int)(g_rng % (uint64_t)(hi - lo + 1));
}

// The addressing of one request does not depend on the others: a shape keeps
// at most 6 of its requests (drawn from its length distributions).
Shape make(const char* name, int B, int W, int hq, int hkv, int ps, int plo, int phi, int tlo,
           int thi) {
  Shape s{name, hkv, hq / hkv, W, ps, {}, {}};
  if (plo < phi) {  // the extremes of the prompt range, then random draws
    s.P.push_back(plo);
    s.T.push_back(thi);
    s.P.push_back(phi);
    s.T.push_back(tlo);
  }
  for (int b = (int)s.P.size(); b < std::min(B, 6); ++b) {
    s.P.push_back(draw(plo, phi));
    s.T.push_back(draw(tlo, thi));
  }
  return s;
}

int log2i(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

// One instantiation: element size 2 (bf16/f16), head_dim D, MB query blocks per
// wave, KT keys per tile, NST stages; tails = the LDS slot-table tail phase.
template <int D, int MB, int KT, int NST>
void check_inst(const char* mode, bool tails, bool one_per_cu, const std::vector<Shape>& shapes,
                std::vector<int> chunks) {
  using TG = bsp::TileGeom<2, D, KT, NST>;
  char tag[160];
  std::snprintf(tag, sizeof(tag), "%s D=%d MB=%d KT=%d NST=%d", mode, D, MB, KT, NST);
  const std::string t(tag);
  // ---- LDS extents: ring + page window + tail table, per workgroup and per CU
  const int lds = TG::RING * 2 + kPageWin * 4 + (tails ? kTailSlots : 1) * 4;
  need(lds <= kLdsPerCu, t + ": LDS per workgroup " + std::to_string(lds));
  need(one_per_cu || 2 * lds <= kLdsPerCu, t + ": two workgroups per CU do not fit the LDS");
  need(TG::NI >= 1 && TG::TILE * 2 % 4096 == 0, t + ": tile does not split into 1 KB loads");
  // ---- tile loads: every (wave, load, lane) puts 16 bytes at a distinct
  // (row, chunk) of the tile, inside the ring
  std::vector<int> seen(KT * TG::CPR, 0);
  for (int stage = 0; stage < NST; ++stage)
    for (int kv = 0; kv < 2; ++kv)
      for (int wave = 0; wave < 4; ++wave)
        for (int i = 0; i < TG::NI; ++i) {
          const int dst = TG::ring_dst(stage, kv, wave, i);
          need(dst >= 0 && dst + TG::EPK <= TG::RING, t + ": ring destination");
          if (stage == 0 && kv == 0)
            for (int lane = 0; lane < 64; ++lane) {
              const int r = TG::load_row(wave, i, lane), c = TG::load_chunk(wave, i, lane);
              need(r >= 0 && r < KT && c >= 0 && c < TG::CPR, t + ": tile row/chunk");
              if (r >= 0 && r < KT && c >= 0 && c < TG::CPR) ++seen[r * TG::CPR + c];
              // the lane fetches logical chunk c of row r and lands it at position
              // c ^ swz(r) of that row, where the operand reads look for it
              need(dst + lane * 8 == r * D + (c ^ TG::swz(r)) * 8, t + ": load lands off its row/chunk");
            }
        }
  for (int x : seen) need(x == 1, t + ": tile chunk written " + std::to_string(x) + " times");
  // ---- operand reads of a tile (S^T: K rows; O^T: V^T transpose reads)
  for (int kb = 0; kb < KT / 16; ++kb)
    for (int l = 0; l < 64; ++l)
      for (int ds = 0; ds < D / 32; ++ds) {
        const int off = TG::k_read(kb * 16 + (l & 15), ds * 4 + (l >> 4));
        need(off >= 0 && off + 8 <= TG::TILE, t + ": K operand read");
      }
  for (int s2 = 0; s2 < KT / 32; ++s2)
    for (int l = 0; l < 64; ++l)
      for (int db = 0; db < D / 16; ++db) {
        const int ra = 32 * s2 + 4 * (l >> 4) + ((l & 15) >> 2);
        const int off = TG::v_read(ra, db * 16 + 4 * (l & 3));
        need(off >= 0 && off + 4 <= TG::TILE && off + 16 * D + 4 <= TG::TILE,
             t + ": V transpose read");
      }
  // ---- tail sub-tiles in each wave's share of the ring
  if (tails) {
    need(TG::REGION >= 2 * TG::SUB && TG::NIW >= 1, t + ": sub-tile larger than a wave's share");
    for (int wave = 0; wave < 4; ++wave)
      for (int buf = 0; buf < TG::NBUF; ++buf)
        for (int kv = 0; kv < 2; ++kv)
          for (int i = 0; i < TG::NIW; ++i) {
            const int dst = TG::region_dst(wave, buf, kv, i);
            need(dst >= wave * TG::REGION && dst + TG::EPK <= (wave + 1) * TG::REGION,
                 t + ": tail sub-tile outside the wave's share");
            for (int lane = 0; lane < 64; ++lane) {
              const int r = TG::sub_row(i, lane), c = TG::sub_chunk(i, lane);
              need(r >= 0 && r < TG::KW && c >= 0 && c < TG::CPR, t + ": sub-tile row/chunk");
              need(dst + lane * 8 == TG::region_dst(wave, buf, kv, 0) + r * D + (c ^ TG::swz(r)) * 8,
                   t + ": sub-tile load lands off its row/chunk");
            }
          }
    for (int l = 0; l < 64; ++l) {
      for (int ds = 0; ds < D / 32; ++ds)
        need(TG::k_read(l & 15, ds * 4 + (l >> 4)) + 8 <= TG::SUB, t + ": tail K read");
      for (int db = 0; db < D / 16; ++db)
        need(TG::v_read(4 * (l >> 4) + ((l & 15) >> 2), db * 16 + 4 * (l & 3)) + 4 <= TG::SUB,
             t + ": tail V read");
    }
  }
  // ---- shapes: page windows, tile loads from the pool, token writes
  for (const Shape& s : shapes) {
    const int shift = log2i(s.ps), pmask = s.ps - 1;
    int64_t pages_used = 0;
    for (size_t b = 0; b < s.P.size(); ++b) pages_used += (s.P[b] + s.ps - 1) / s.ps + s.W * 2;
    const int64_t num_pages = pages_used + 1;
    const int64_t pool = num_pages * s.hkv * s.ps * (int64_t)D;
    const std::string ts = t + " shape " + s.name;
    const int rows = s.W * s.group;
    if (tails) {  // the launcher takes this mode only when the tails fit the table
      const int nbt_max = std::min(s.W, (64 * MB - 1) / s.group + 2);
      int tmax = 0;
      for (int x : s.T) tmax = std::max(tmax, x);
      if ((int64_t)nbt_max * tmax <= kTailSlots)
        for (int qt = 0; qt * 64 * MB < rows; ++qt) {
          const int kb_first = qt * 64 * MB / s.group;
          const int kb_last = std::min(s.W - 1, ((qt + 1) * 64 * MB - 1) / s.group);
          need((int64_t)(kb_last - kb_first + 1) * tmax <= kTailSlots, ts + ": slot table");
        }
    }
    for (size_t b = 0; b < s.P.size(); ++b) {
      for (int ck : chunks) {  // whole prompt (0) or split into chunks of ck keys
        const int P = s.P[b];
        const int parts = ck > 0 && P > ck ? (P + ck - 1) / ck : 1;
        for (int part = 0; part < parts; ++part) {
          const int k_lo = parts > 1 ? part * ck : 0;
          const int k_hi = parts > 1 ? std::min(P, (part + 1) * ck) : P;
          const int keys_per_win = kPageWin << shift;
          const int win_first = k_lo / keys_per_win;
          const int n_win = k_hi > k_lo ? (k_hi - 1) / keys_per_win - win_first + 1 : 0;
          for (int wi = 0; wi < n_win; ++wi) {
            const int w0 = (win_first + wi) * keys_per_win;
            const int seg_lo = std::max(k_lo, w0), seg_hi = std::min(k_hi, w0 + keys_per_win);
            const int pg0 = w0 >> shift;
            const int npg = ((std::min(k_hi, w0 + keys_per_win) - 1) >> shift) - pg0 + 1;
            need(npg >= 1 && npg <= kPageWin, ts + ": page window size");
            const int ntp = (seg_hi - seg_lo + KT - 1) / KT;
            for (int tile = 0; tile < ntp; ++tile) {
              const int t0 = seg_lo + tile * KT;
              const bool one_page = (t0 & pmask) + KT <= pmask + 1;
              for (int wave = 0; wave < 4; ++wave)
                for (int i = 0; i < TG::NI; ++i)
                  for (int lane = 0; lane < 64; ++lane) {
                    const int r = TG::load_row(wave, i, lane), c = TG::load_chunk(wave, i, lane);
                    int j = t0 + r;
                    if (j >= seg_hi) j = t0;
                    const int slot = bsp::window_slot(one_page ? t0 : j, shift, pg0);
                    need(slot >= 0 && slot < npg, ts + ": page id read outside the filled window");
                    for (int ext = 0; ext < 2; ++ext) {  // lowest and highest page and head
                        const int64_t page = ext ? num_pages - 1 : 0;
                        const int g = ext ? s.hkv - 1 : 0;
                        const int64_t off =
                            one_page ? bsp::pool_row(page, s.hkv, g, shift, t0 & pmask, D) +
                                           (int64_t)(t0 + r < seg_hi ? r : 0) * D + c * 8
                                     : bsp::pool_row(page, s.hkv, g, shift, j & pmask, D) + c * 8;
                        need(off >= 0 && off + 8 <= pool, ts + ": tile load outside the pool");
                        if (one_page)  // the scalar-base form stays inside the tile's page
                          need((t0 & pmask) + (t0 + r < seg_hi ? r : 0) < s.ps,
                               ts + ": one-page tile crosses its page");
                      }
                  }
            }
          }
        }
      }
      // token write of the current token (position S - 1 = P + T - 1)
      if (s.T[b] > 0) {
        const int j = s.P[b] + s.T[b] - 1;
        for (int64_t page : {int64_t(0), num_pages - 1})
          for (int g : {0, s.hkv - 1})
            for (int c = 0; c < D / 8; ++c) {
              const int64_t dst = bsp::pool_row(page, s.hkv, g, shift, j & pmask, D) + c * 8;
              need(dst >= 0 && dst + 8 <= pool, ts + ": token write outside the pool");
            }
      }
    }
  }
}

}  // namespace

int main(int argc, char** argv) {
  const bool dropped = argc > 1 && std::string(argv[1]) == "--dropped-d256";
  std::vector<Shape> beam = {
      make("qwen3_0p6b", 64, 30, 16, 8, 32, 400, 600, 0, 4),
      make("wide_beam", 128, 96, 16, 8, 32, 2800, 3200, 0, 8),
      make("qwen3_4b", 64, 30, 32, 8, 32, 1600, 2400, 1, 4),
      make("nsample", 64, 16, 16, 8, 32, 400, 600, 8, 32),
      make("tiny", 1, 4, 2, 1, 16, 128, 128, 3, 3),
      make("groups", 2, 7, 16, 2, 16, 70, 150, 0, 5),
      make("query_tiles", 2, 150, 4, 2, 16, 40, 400, 1, 6),
      make("long_tails", 1, 192, 2, 2, 16, 30, 300, 17, 20),
      make("page_size_1", 2, 6, 4, 2, 1, 40, 400, 1, 5),
      make("page_size_1024", 2, 6, 8, 2, 1024, 300, 2100, 1, 5),
      make("empty_prompts", 3, 5, 4, 2, 16, 0, 0, 1, 6),
      make("cached_decode", 1, 1, 24, 8, 32, 0, 10368, 0, 0),
      make("prefill_rows", 8, 1, 16, 8, 32, 1, 2500, 0, 0),
  };
  const std::vector<int> chunks = {0, 64, 192, 1024};
  if (dropped) {
    // the D = 256, two-block, 64-key, two-stage variant that was never shipped
    check_inst<256, 2, 64, 2>("dropped fused", true, true, beam, chunks);
  } else {
    // bsp_decode_step, tails through the LDS table (launch_mfma, MODE 1)
    check_inst<64, 1, 64, 4>("fused", true, false, beam, chunks);
    check_inst<64, 2, 64, 4>("fused", true, false, beam, chunks);
    check_inst<64, 3, 64, 4>("fused", true, false, beam, chunks);
    check_inst<128, 1, 64, 2>("fused", true, false, beam, chunks);
    check_inst<128, 2, 64, 2>("fused", true, false, beam, chunks);
    check_inst<128, 3, 32, 4>("fused", true, false, beam, chunks);
    check_inst<256, 1, 32, 2>("fused", true, false, beam, chunks);
    // long tails resolved key by key (MODE 2) and the partial-state kernel (MODE 0)
    check_inst<128, 1, 32, 4>("fused long tails / prefix", false, false, beam, chunks);
    check_inst<128, 2, 32, 4>("fused long tails / prefix", false, false, beam, chunks);
    // the context prefill (MODE 3) and the mixed step (MODE 4)
    check_inst<256, 2, 32, 4>("prefill", false, true, beam, {0});
    check_inst<64, 1, 64, 4>("mixed", true, false, beam, {0});
    check_inst<128, 1, 64, 2>("mixed / two-plan", true, false, beam, {0});
  }
  std::printf("%ld checks, %ld out of range\n", g_checks, g_bad);
  return g_bad == 0 ? 0 : 1;
}
