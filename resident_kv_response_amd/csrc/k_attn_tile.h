// Tile geometry and LDS staging shared by the bf16 MFMA attention kernels (gfx950).
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

template <int D>
struct TileCfg {
  static constexpr int WAVES = 4;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int NT = 2;                    // 32-row N-tiles per wave
  static constexpr int ROWS_W = 32 * NT;          // query rows per wave
  static constexpr int BM = WAVES * ROWS_W;       // query rows per workgroup
  static constexpr int BN = 64;                   // keys per LDS stage
  static constexpr int KS = D / 16;               // k-steps of a contraction over d
  static constexpr int DT = D / 32;               // 32-wide d-tiles of an output over d
  static constexpr int ROW = D + 8;               // padded bf16 row: [key][d] tiles
  static constexpr int TROW = BN + 8;             // padded bf16 row: [d][key] tiles
  static constexpr int NORM_ELEMS = BN * ROW;     // one [BN][D] tile
  static constexpr int TRANS_ELEMS = D * TROW;    // one [D][BN] tile
  // global -> LDS staging work per tile
  static constexpr int PIECES = BN * (D / 8);         // 16-byte pieces of a [BN][D] tile
  static constexpr int QUADS = (BN / 4) * (D / 8);    // (4 keys x 8 dims) blocks
  static constexpr int PIECES_PER_THREAD = (PIECES + THREADS - 1) / THREADS;
  static constexpr int QUADS_PER_THREAD = (QUADS + THREADS - 1) / THREADS;
};

// 16-byte global load of keys [key0, key_end) of a K or V stream; zeros past the end.
__device__ __forceinline__ uint4 load_row16(const uint16_t* base, int64_t key, int64_t key_end,
                                            int64_t stride, int col) {
  if (key < key_end) return *reinterpret_cast<const uint4*>(base + key * stride + col);
  return make_uint4(0u, 0u, 0u, 0u);
}

// Registers holding one tile in flight between global memory and LDS.
template <int D, int NP>
struct RowPieces {
  uint4 v[NP];
};

template <int D, int NQ>
struct QuadPieces {
  uint4 v[NQ][4];
};

// Load a [BN][D] tile as plain 16-byte pieces (thread-strided).
template <int D>
__device__ __forceinline__ void load_pieces(RowPieces<D, TileCfg<D>::PIECES_PER_THREAD>& rp,
                                            const uint16_t* base, int64_t key0, int64_t key_end,
                                            int64_t stride) {
  using C = TileCfg<D>;
#pragma unroll
  for (int i = 0; i < C::PIECES_PER_THREAD; ++i) {
    const int p = threadIdx.x + i * C::THREADS;
    const int key = p / (D / 8), col = (p % (D / 8)) * 8;
    rp.v[i] = (p < C::PIECES) ? load_row16(base, key0 + key, key_end, stride, col) : make_uint4(0, 0, 0, 0);
  }
}

template <int D>
__device__ __forceinline__ void store_pieces(const RowPieces<D, TileCfg<D>::PIECES_PER_THREAD>& rp,
                                             uint16_t* tile) {
  using C = TileCfg<D>;
#pragma unroll
  for (int i = 0; i < C::PIECES_PER_THREAD; ++i) {
    const int p = threadIdx.x + i * C::THREADS;
    if (p < C::PIECES) {
      const int key = p / (D / 8), col = (p % (D / 8)) * 8;
      *reinterpret_cast<uint4*>(tile + key * C::ROW + col) = rp.v[i];
    }
  }
}

// Load a [BN][D] tile as (4 consecutive keys x 8 dims) blocks, for a transposed store.
template <int D>
__device__ __forceinline__ void load_quads(QuadPieces<D, TileCfg<D>::QUADS_PER_THREAD>& qp,
                                           const uint16_t* base, int64_t key0, int64_t key_end,
                                           int64_t stride) {
  using C = TileCfg<D>;
#pragma unroll
  for (int i = 0; i < C::QUADS_PER_THREAD; ++i) {
    const int p = threadIdx.x + i * C::THREADS;
    const int kq = p / (D / 8), col = (p % (D / 8)) * 8;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      qp.v[i][u] = (p < C::QUADS) ? load_row16(base, key0 + 4 * kq + u, key_end, stride, col)
                                  : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ uint32_t word_of(const uint4& v, int w) {
  return w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
}

// Transposed store: tile[d][pos(key)] with keys permuted inside each 32-group (swap23).
template <int D>
__device__ __forceinline__ void store_quads_transposed(
    const QuadPieces<D, TileCfg<D>::QUADS_PER_THREAD>& qp, uint16_t* tile) {
  using C = TileCfg<D>;
#pragma unroll
  for (int i = 0; i < C::QUADS_PER_THREAD; ++i) {
    const int p = threadIdx.x + i * C::THREADS;
    if (p >= C::QUADS) continue;
    const int kq = p / (D / 8), col = (p % (D / 8)) * 8;
    const int key = 4 * kq;
    const int pos = (key & ~31) | swap23(key & 31);
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      const int w = dd >> 1;
      const uint32_t a0 = word_of(qp.v[i][0], w), a1 = word_of(qp.v[i][1], w);
      const uint32_t a2 = word_of(qp.v[i][2], w), a3 = word_of(qp.v[i][3], w);
      uint2 out;
      if (dd & 1) {
        out.x = (a0 >> 16) | (a1 & 0xFFFF0000u);
        out.y = (a2 >> 16) | (a3 & 0xFFFF0000u);
      } else {
        out.x = (a0 & 0xFFFFu) | (a1 << 16);
        out.y = (a2 & 0xFFFFu) | (a3 << 16);
      }
      *reinterpret_cast<uint2*>(tile + (col + dd) * C::TROW + pos) = out;
    }
  }
}

// Plain store of the quads (for tiles needed both plain and transposed).
template <int D>
__device__ __forceinline__ void store_quads_plain(
    const QuadPieces<D, TileCfg<D>::QUADS_PER_THREAD>& qp, uint16_t* tile) {
  using C = TileCfg<D>;
#pragma unroll
  for (int i = 0; i < C::QUADS_PER_THREAD; ++i) {
    const int p = threadIdx.x + i * C::THREADS;
    if (p >= C::QUADS) continue;
    const int kq = p / (D / 8), col = (p % (D / 8)) * 8;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      *reinterpret_cast<uint4*>(tile + (4 * kq + u) * C::ROW + col) = qp.v[i][u];
  }
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
