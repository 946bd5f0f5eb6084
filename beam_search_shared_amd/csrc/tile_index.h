// Address arithmetic of the shared-key kernel (prefix_attn.hip), as host-and-
// device functions: the kernel computes every LDS and global offset of its
// tile ring, tail sub-tiles, operand reads and token writes through these, and
// a CPU model (tests/index_model.cpp) drives the same functions over every
// instantiation the library ships, to show each offset inside its buffer.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace bsp {

// Geometry of one kernel instantiation: element size ESZ (bytes), head_dim D,
// KT keys per tile, NST stages in the ring.
template <int ESZ, int D, int KT, int NST>
struct TileGeom {
  static constexpr int CPR = D / 8;              // 16-byte chunks per key row
  static constexpr int TILE = KT * D;            // elements of K (or V) per tile
  static constexpr int EPK = 1024 / ESZ;         // elements per 1 KB wave load
  static constexpr int NI = TILE * ESZ / 4096;   // 1 KB loads per wave per tile (K, and V)
  static constexpr int RING = NST * 2 * TILE;    // elements of the K/V ring
  static constexpr int KW = 16;                  // keys per tail sub-tile
  static constexpr int SUB = KW * D;             // elements of K (or V) per sub-tile
  static constexpr int NIW = SUB * ESZ / 1024;   // 1 KB loads per sub-tile (K, and V)
  static constexpr int REGION = RING / 4;        // elements of each wave's share of the ring
  static constexpr int NBUF = REGION >= 4 * SUB ? 2 : 1;  // tail sub-tile buffers per wave

  // XOR swizzle of the 16-byte chunks of a key row in LDS (a function of the
  // low 4 row bits): chunk c of row r is stored at chunk c ^ swz(r). It keeps
  // the K-operand reads (16 consecutive rows, one chunk each) and the V
  // transpose reads (4 rows x 2 chunks per 16 lanes) on distinct banks.
  static __host__ __device__ __forceinline__ int swz(int r) {
    const int a = ((r & 1) << 1) ^ ((r & 2) << 1) ^ ((r >> 3) & 1);
    return a ^ ((r & 4) ? (D == 64 ? 3 : 9) : 0);
  }
  // Tile load i of wave `wave`: lane `lane` moves 16 bytes of tile row
  // load_row() into swizzled chunk load_chunk(); the wave's 1 KB lands at ring
  // element ring_dst() (stage, kv: 0 K, 1 V).
  static __host__ __device__ __forceinline__ int load_row(int wave, int i, int lane) {
    return ((wave * NI + i) * 64 + lane) / CPR;
  }
  static __host__ __device__ __forceinline__ int load_chunk(int wave, int i, int lane) {
    const int chunk = (wave * NI + i) * 64 + lane;
    return (chunk % CPR) ^ swz(chunk / CPR);
  }
  static __host__ __device__ __forceinline__ int ring_dst(int stage, int kv, int wave, int i) {
    return (stage * 2 + kv) * TILE + (wave * NI + i) * EPK;
  }
  // K operand (S^T = K Q^T): element of a K tile that lane (row r, 8-element
  // column chunk cc) reads as 16 bytes.
  static __host__ __device__ __forceinline__ int k_read(int r, int cc) {
    return r * D + ((cc ^ swz(r)) << 3);
  }
  // V^T operand (transpose read): element of a V tile at which the 8-byte read
  // of row ra, column col starts.
  static __host__ __device__ __forceinline__ int v_read(int ra, int col) {
    return ra * D + ((((col >> 3) ^ swz(ra)) << 3) + (col & 7));
  }
  // Tail sub-tiles: wave `wave`'s buffer `buf` in its share of the ring; load
  // i puts lane `lane`'s 16 bytes of sub-tile row sub_row() at chunk
  // sub_chunk(); the 1 KB of K (kv 0) or V (kv 1) lands at region_dst().
  static __host__ __device__ __forceinline__ int sub_row(int i, int lane) {
    return (i * 64 + lane) / CPR;
  }
  static __host__ __device__ __forceinline__ int sub_chunk(int i, int lane) {
    const int chunk = i * 64 + lane;
    return (chunk % CPR) ^ swz(chunk / CPR);
  }
  static __host__ __device__ __forceinline__ int region_dst(int wave, int buf, int kv, int i) {
    return wave * REGION + buf * 2 * SUB + kv * SUB + i * EPK;
  }
};

// Element offset of row `row` of KV head g in page `page` of a pool
// [pages][hkv][1 << shift][D].
__host__ __device__ __forceinline__ int64_t pool_row(int64_t page, int hkv, int g, int shift,
                                                     int row, int D) {
  return (((page * hkv + g) << shift) + row) * (int64_t)D;
}

// Index of key j's page id in the LDS window whose first page is pg0.
__host__ __device__ __forceinline__ int window_slot(int j, int shift, int pg0) {
  return (j >> shift) - pg0;
}

}  // namespace bsp
