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

__device__ __forceinline__ TileWork decode_tile_work(const Geom& g, int BM) {
  TileWork w;
  const int64_t m_lo = (int64_t)g.row_lo * g.grp, m_hi = (int64_t)g.row_hi * g.grp;
  const int64_t n_mt = (m_hi - m_lo + BM - 1) / BM;
  const int64_t n_work = (int64_t)g.K * g.Hkv * g.n_parts * n_mt;
  int64_t idx = xcd_work_index(n_work);
  w.ok = idx >= 0;
  if (!w.ok) return w;
  const int64_t mt = idx % n_mt;
  idx /= n_mt;
  w.part = (int)(idx % g.n_parts);
  idx /= g.n_parts;
  w.g = (int)(idx % g.Hkv);
  w.k = (int)(idx / g.Hkv);
  w.m0 = (int)(m_lo + mt * BM);
  return w;
}

inline int64_t tile_work_count(const Geom& g, int BM) {
  const int64_t m = (int64_t)(g.row_hi - g.row_lo) * g.grp;
  return (int64_t)g.K * g.Hkv * g.n_parts * ((m + BM - 1) / BM);
}

}  // namespace rr
