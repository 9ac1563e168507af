// Tile geometry shared by the bf16 MFMA attention kernels (gfx950).
//
// MFMA v_mfma_f32_32x32x16_bf16 operand layout (wave64, lane l, h = l / 32):
//   A (32 x 16):  lane l holds A[l % 32][8h .. 8h+7]
//   B (16 x 32):  lane l holds B[8h .. 8h+7][l % 32]
//   C (32 x 32):  lane l, register i holds C[8(i/4) + 4h + (i%4)][l % 32]
// The kernels compute score tiles transposed, S^T = K Q^T (keys x rows), so that each
// lane owns one query row (column l % 32) and 16 of the tile's 32 keys.  Row statistics
// then need one exchange with lane l ^ 32 only, and the C registers of S^T are directly
// the B operand of the next contraction over keys (P^T or dS^T), provided the key order
// inside each 32-key group is permuted consistently on the A side: C register i = 8s + j
// of lane half h holds key 16s + 8(j/4) + 4h + (j%4), i.e. the key with bits 2 and 3 of
// its index swapped relative to the MFMA k-slot 16s + 8h + j.  Transposed LDS tiles store
// keys at that swapped position so every A fragment is one 16-byte LDS read.
#pragma once

#include "k_common.h"

namespace rr {

// Position of key (or row) x of a 32-group inside a transposed LDS tile: bits 2 and 3
// swapped.
__device__ __forceinline__ int swap23(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// 32-bit word w of a 16-byte vector.
__device__ __forceinline__ uint32_t word_of(const uint4& v, int w) {
  return w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
}

// Work item of the query-parallel kernels: (response k, KV head g, part, row tile).
struct TileWork {
  int k, g, part;
  int m0;      // first flattened row (r * grp + hh) of the workgroup
  bool ok;
};

// Row tiles of response k inside the launch's row range: only rows below r_len[k] get a
// workgroup, so responses shorter than the stride R_max cost nothing for their padding.
__host__ __device__ __forceinline__ int64_t member_tiles(const Geom& g, int k, int BM) {
  const int hi = g.r_len[k] < g.row_hi ? g.r_len[k] : g.row_hi;
  const int64_t m = hi > g.row_lo ? (int64_t)(hi - g.row_lo) * g.grp : 0;
  return (m + BM - 1) / BM;
}

__host__ __device__ __forceinline__ int64_t tiles_per_part(const Geom& g, int BM) {
  int64_t t = 0;
  for (int k = 0; k < g.K; ++k) t += member_tiles(g, k, BM);
  return t;
}

// Work order: (KV head, part) outermost, then every response's row tiles.  Consecutive
// work items (which xcd_work_index keeps on one XCD) read the same prompt chunk, and each
// XCD receives an equal share of real tiles whatever the spread of response lengths.
__device__ __forceinline__ TileWork decode_tile_work(const Geom& g, int BM) {
  TileWork w;
  const int64_t T = tiles_per_part(g, BM);
  const int64_t n_work = (int64_t)g.Hkv * g.n_parts * T;
  int64_t idx = xcd_work_index(n_work);
  w.ok = idx >= 0;
  if (!w.ok) return w;
  int64_t j = idx % T;
  idx /= T;
  w.part = (int)(idx % g.n_parts);
  w.g = (int)(idx / g.n_parts);
  int k = 0;
  for (int64_t t = member_tiles(g, 0, BM); j >= t; t = member_tiles(g, ++k, BM)) j -= t;
  w.k = k;
  w.m0 = (int)((int64_t)g.row_lo * g.grp + j * BM);
  return w;
}

inline int64_t tile_work_count(const Geom& g, int BM) {
  return (int64_t)g.Hkv * g.n_parts * tiles_per_part(g, BM);
}

}  // namespace rr
