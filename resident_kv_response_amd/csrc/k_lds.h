// LDS staging for the bf16 MFMA attention kernels (gfx950): direct global->LDS loads of
// row-major [rows][D] bf16 tiles with an XOR swizzle, and the two fragment reads the
// kernels need from such a tile.
//
// Swizzle: a row is D/8 16-byte granules; logical granule g of row r is stored at
// granule g ^ f(r).  Rows are not padded, so a wave-wide direct load (64 lanes x 16 bytes,
// stored at consecutive LDS addresses) fills whole rows.  With D = 128 a row spans all 64
// banks, and f(r) = ((r & 3) << 2) | ((r >> 2) & 3) is a bijection on r mod 16: the 16
// consecutive rows of a 128-bit row-fragment read land on 16 different granules, and the
// four consecutive rows x four granules of a half-wave transposing read cover all 16
// granules once.  With D = 64 two rows share the 64 banks and f(r) = (r >> 1) & 7.
//
// Fragment reads (lane l, h = l / 32, wave64):
//   row fragment     A[m][k] = T[row0 + l%32][16*ks + 8h .. +8]      one ds_read_b128
//   transposed frag  A[m][k] = T[row(k)][col0 + l%32], 8 rows per lane  two ds_read_b64_tr_b16
// ds_read_b64_tr_b16 semantics (gfx950): in each 16-lane group, result lane r, element j
// is element (r % 4) of the 64-bit chunk addressed by lane 4j + r/4 of the group.  If lane
// i of the group addresses T[base + i/4][c0 + 4(i%4) .. +4], result lane r gets
// T[base + j][c0 + r] for j = 0..3: four consecutive rows of its own column.
#pragma once

#include "k_addr.h"
#include "k_common.h"

namespace rr {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <int D>
struct Swz {
  static constexpr int G = D / 8;        // granules per row
  static constexpr int ROW_BYTES = D * 2;
  static __device__ __forceinline__ int f(int r) { return swz(D, r); }
  // byte offset of logical granule g of row r
  static __device__ __forceinline__ int off(int r, int g) { return r * ROW_BYTES + ((g ^ f(r)) << 4); }
};

// Direct loads of a [N_ROWS][D] tile.  Row r of the tile comes from byte offset
// r * stride_bytes of `src` (a wave-uniform base, so the load takes a scalar base plus a
// 32-bit lane offset).  Each of the workgroup's waves issues PER_WAVE wave-wide loads of
// 64 x 16 bytes, which land at consecutive LDS addresses.
template <int D, int N_ROWS, int WAVES>
struct DirectLoad {
  static constexpr int G = D / 8;                       // granules per row
  static constexpr int RPI = 64 / G;                    // rows per wave instruction
  static constexpr int GRAN = N_ROWS * G;
  static constexpr int PER_WAVE = GRAN / (64 * WAVES);
  static_assert(GRAN % (64 * WAVES) == 0, "tile must split evenly over the waves");
  static_assert(RPI == 4 || RPI == 8, "D must be 128 or 64");

  TileLoadPre pre;      // per-lane constants (k_addr.h)

  __device__ __forceinline__ void init(int64_t stride_bytes) {
    pre = tile_load_pre(D, N_ROWS, WAVES, threadIdx.x >> 6, threadIdx.x & 63, stride_bytes);
  }
  // tile rows [0, N_ROWS) <- rows src_row0 .. of the stream; rows at or past row_end are
  // redirected to row_end - 1 (their values are masked by the caller).  Requires
  // src_row0 < row_end.  Addresses from tile_load_at (k_addr.h).
  __device__ __forceinline__ void issue(char* tile, const uint16_t* stream, int64_t src_row0,
                                        int64_t row_end, int64_t stride_bytes) const {
    const char* sbytes = reinterpret_cast<const char*>(stream);
    const bool full = src_row0 + N_ROWS <= row_end;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const TileLoadAt a = tile_load_at(pre, D, i, src_row0, row_end, stride_bytes, full);
      __builtin_amdgcn_global_load_lds(sbytes + a.src_off, (lds_void*)(tile + a.lds_base), 16, 0, 0);
    }
  }
};

// Direct loads of a [N_ROWS][D] tile for the ring kernels: tile rows [0, N_ROWS) <- rows of
// a stream whose row 0 starts at the wave-uniform address `base`; rows at or past
// `rows_valid` (>= 1) re-read row rows_valid - 1 (their values are masked by the caller).
// Only the base is 64-bit; lane offsets are 32-bit, so N_ROWS * stride_bytes must stay
// below 2^31.  The destination is a LDS byte address (see lds_addr).  Addresses from
// rows_load_pre / rows_load_at (k_addr.h).
//
// The loads are issued from inline assembly (M0 = the wave's LDS destination, then
// global_load_lds_dwordx4 with a scalar base and a 32-bit lane offset).  The compiler
// then does not track them, and callers order them explicitly: s_waitcnt vmcnt before
// the barrier that publishes a stage, and no load into a buffer that a wave may still
// read.  (When the compiler does track them it treats every outstanding LDS read as
// unordered and waits for all of them before each use, which defeats reading fragments
// ahead.)
template <int D, int N_ROWS, int WAVES>
struct DirectLoadRows {
  using DL = DirectLoad<D, N_ROWS, WAVES>;
  static constexpr int G = DL::G, RPI = DL::RPI, PER_WAVE = DL::PER_WAVE;
  RowsLoadPre pre;      // per-lane constants (k_addr.h)

  __device__ __forceinline__ void init() {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    pre = rows_load_pre(D, N_ROWS, WAVES, wave, threadIdx.x & 63);
  }
  __device__ __forceinline__ void issue(uint32_t tile_lds, const char* base, int rows_valid,
                                        uint32_t stride_bytes) const {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const RowsLoadAt a = rows_load_at(pre, D, i, rows_valid, stride_bytes);
      const uint32_t lds = tile_lds + a.lds_base;
      asm volatile(
          "s_mov_b32 m0, %0\n\t"
          "s_nop 0\n\t"
          "global_load_lds_dwordx4 %1, %2"
          :
          : "s"(lds), "v"(a.src_off), "s"(base)
          : "memory", "m0");
    }
  }
};

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Fragment reads from a swizzled [rows][D] tile.  Every read address is a per-lane
// offset computed once (the swizzle depends only on the row mod 16, and the subtile and
// half-subtile row offsets used below are multiples of 16 rows) plus a compile-time
// offset, so the reads need no address arithmetic in the loop.
template <int D>
struct Frag {
  static constexpr int KS = D / 16, DT = D / 32, ROW = D * 2;
  uint32_t rows[KS];        // row fragment, k-step ks, subtile 0
  uint32_t trans[DT][2];    // transposed fragment, d-tile dt, rows +0 / +8, subtile 0

  __device__ __forceinline__ void init() {
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int r = lane & 31;
      rows[ks] = (uint32_t)(r * ROW + (((2 * ks + h) ^ Swz<D>::f(r)) << 4));
    }
    const int i = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int r = 4 * h + (i >> 2) + 8 * hi;
        const int c = 32 * dt + 16 * (grp & 1) + 4 * (i & 3);   // element column of the chunk
        trans[dt][hi] = (uint32_t)(r * ROW + (((c >> 3) ^ Swz<D>::f(r)) << 4) + (c & 7) * 2);
      }
  }

  // Row fragment: lane holds T[32*sub + l%32][16*ks + 8h .. +8].
  __device__ __forceinline__ bf16x8 row(const char* tile, int sub, int ks) const {
    return *reinterpret_cast<const bf16x8*>(tile + rows[ks] + sub * 32 * ROW);
  }

  // Lane offsets (rows +0 / +8) of the transposed fragment at a run-time column offset
  // col0 (a multiple of 32), for callers whose column tile is not a compile-time index.
  static __device__ __forceinline__ void trans_offsets(int col0, uint32_t (&off)[2]) {
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5, i = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int r = 4 * h + (i >> 2) + 8 * hi;
      const int c = col0 + 16 * (grp & 1) + 4 * (i & 3);
      off[hi] = (uint32_t)(r * ROW + (((c >> 3) ^ Swz<D>::f(r)) << 4) + (c & 7) * 2);
    }
  }
  static __device__ __forceinline__ bf16x8 trans_at(const char* tile, const uint32_t (&off)[2], int sub, int h2) {
    const int rb = (sub * 32 + 16 * h2) * ROW;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + off[0] + rb));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + off[1] + rb));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  }

  // Transposed fragment: A[m][k] = T[row(k)][32*dt + l%32] with k-slots 0..3 <- rows
  // 32*sub + 16*h2 + 4h + 0..3 and k-slots 4..7 <- rows 32*sub + 16*h2 + 8 + 4h + 0..3
  // (h = l/32).  This is the key order of the MFMA C layout, so the fragment pairs with
  // P^T / dS^T taken straight from the C registers of a 32x32 score tile.
  __device__ __forceinline__ bf16x8 trans_frag(const char* tile, int sub, int h2, int dt) const {
    const int rb = (sub * 32 + 16 * h2) * ROW;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + trans[dt][0] + rb));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + trans[dt][1] + rb));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  }
};

// s_waitcnt vmcnt(0) leaving the other counters alone (gfx9 encoding).
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// max of a value over lanes l and l ^ 32
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace rr
