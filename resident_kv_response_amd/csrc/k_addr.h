// Integer address arithmetic of the direct global->LDS tile loads (k_lds.h), as plain
// constexpr functions on integers.  The kernels compute every load address through them,
// and tests/native/host_checks.cpp, compiled for the host, checks them over every tile
// shape and stage length the kernels use: each load stays inside the stage's rows, and
// each LDS granule receives the row and granule the fragment reads expect.
//
// A tile is [n_rows][D] bf16, D/8 granules of 16 bytes per row, stored with an XOR
// swizzle: logical granule g of tile row r sits at granule position g ^ swz(D, r).  A wave
// instruction moves 64 lanes x 16 bytes to 1 KiB of consecutive LDS: lane l writes tile
// row (first row of the instruction) + l / G, granule position l % G, so it must read
// source granule (l % G) ^ swz(D, row).
#pragma once

#include <stdint.h>

namespace rr {

constexpr int swz(int D, int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((r >> 1) & 7);
}

// Per-lane constants of the ring kernels' stage loads (DirectLoadRows): wave `wave` of
// `waves` issues PER_WAVE = n_rows * G / (64 * waves) instructions; instruction i covers
// tile rows row0 + RPI * i + [0, RPI).  gran[i & 3] is the lane's source granule byte
// offset for instruction i (the swizzle repeats every 16 rows, and four instructions
// advance 4 * RPI rows, a multiple of 16).
struct RowsLoadPre {
  int row0;          // first tile row of the wave
  int r_lane;        // row of the lane inside an instruction
  uint32_t lds0;     // LDS byte offset of the wave's first granule in the tile
  uint32_t gran[4];  // source granule byte offset within a row, by instruction index mod 4
};

constexpr RowsLoadPre rows_load_pre(int D, int n_rows, int waves, int wave, int lane) {
  const int G = D / 8, RPI = 64 / G;
  const int per_wave = n_rows * G / (64 * waves);
  RowsLoadPre p{};
  p.row0 = wave * per_wave * RPI;
  p.r_lane = lane / G;
  p.lds0 = (uint32_t)(p.row0 / RPI) * 64u * 16u;
  for (int par = 0; par < 4; ++par) {
    const int r = p.row0 + RPI * par + p.r_lane;
    p.gran[par] = (uint32_t)(((lane % G) ^ swz(D, r)) << 4);
  }
  return p;
}

// Instruction i of a stage whose rows [0, rows_valid) exist (rows_valid >= 1): the lane's
// source byte offset from the stage base (rows at or past rows_valid re-read row
// rows_valid - 1; 32-bit, so 64 * stride_bytes must stay below 2^31) and its LDS byte
// offset in the tile.
struct RowsLoadAt {
  int tile_row;      // tile row the lane's 16 bytes land in
  int src_row;       // stage row they are read from
  uint32_t src_off;  // byte offset from the stage base
  uint32_t lds_base; // byte offset in the tile of the instruction's 1 KiB (wave-uniform);
                     // lane l writes lds_base + 16 l
};

constexpr RowsLoadAt rows_load_at(const RowsLoadPre& p, int D, int i, int rows_valid, uint32_t stride_bytes) {
  const int G = D / 8, RPI = 64 / G;
  RowsLoadAt a{};
  a.tile_row = p.row0 + RPI * i + p.r_lane;
  a.src_row = a.tile_row < rows_valid - 1 ? a.tile_row : rows_valid - 1;
  a.src_off = (uint32_t)a.src_row * stride_bytes + p.gran[i & 3];
  a.lds_base = p.lds0 + (uint32_t)i * 64u * 16u;
  return a;
}

// The same for the general tile loads (DirectLoad), whose stage may begin anywhere in a
// long stream: a 64-bit source row index, rows at or past row_end re-read row_end - 1.
struct TileLoadPre {
  int row0;          // first tile row of the wave
  int r_lane;        // row of the lane inside an instruction
  uint32_t voff[4];  // lane byte offset within an instruction's rows, by index mod 4
};

constexpr TileLoadPre tile_load_pre(int D, int n_rows, int waves, int wave, int lane, int64_t stride_bytes) {
  const int G = D / 8, RPI = 64 / G;
  const int per_wave = n_rows * G / (64 * waves);
  TileLoadPre p{};
  p.row0 = wave * per_wave * RPI;
  p.r_lane = lane / G;
  for (int par = 0; par < 4; ++par) {
    const int r = p.row0 + RPI * par + p.r_lane;
    const int g = (lane % G) ^ swz(D, r);
    p.voff[par] = (uint32_t)((lane / G) * stride_bytes + g * 16);
  }
  return p;
}

struct TileLoadAt {
  int64_t src_row;   // stream row read
  int64_t src_off;   // byte offset from the stream base
  uint32_t lds_base; // byte offset in the tile of the instruction's 1 KiB (wave-uniform);
                     // lane l writes lds_base + 16 l
};

// Instruction i for tile rows [0, n_rows) <- stream rows src_row0 + ..., requires
// src_row0 < row_end.  `full` (src_row0 + n_rows <= row_end) takes the unclamped form.
constexpr TileLoadAt tile_load_at(const TileLoadPre& p, int D, int i, int64_t src_row0, int64_t row_end,
                                  int64_t stride_bytes, bool full) {
  const int G = D / 8, RPI = 64 / G;
  TileLoadAt a{};
  const int64_t r_first = src_row0 + p.row0 + RPI * i;
  if (full) {
    a.src_row = r_first + p.r_lane;
    a.src_off = r_first * stride_bytes + p.voff[i & 3];
  } else {
    const int64_t want = r_first + p.r_lane;
    a.src_row = want < row_end - 1 ? want : row_end - 1;
    const uint32_t gran = p.voff[i & 3] - (uint32_t)(p.r_lane * stride_bytes);   // g * 16
    a.src_off = a.src_row * stride_bytes + gran;
  }
  a.lds_base = (uint32_t)(p.row0 / RPI + i) * 64u * 16u;
  (void)G;
  return a;
}

}  // namespace rr
