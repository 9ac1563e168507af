// Helpers shared by the ring-pipelined MFMA kernels (gfx950): a ring of four LDS stages
// holds K and V tiles as separate arrays, K tiles below 64 KiB and V tiles above.
#pragma once

#include "k_lds.h"

namespace rr {

// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding, n < 16).
template <int N>
__device__ __forceinline__ void wait_vmcnt_n() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Lane offsets of fragment reads from tiles that lie above the 16-bit immediate offset
// range of a LDS read.  The offsets are biased by 2^16 and hidden from the compiler, so
// every such tile is reached as (one set of offset registers) + immediate instead of one
// register set per tile.
template <int D>
struct FarFrags {
  static constexpr uint32_t kBias = 1u << 16;
  uint32_t rows[D / 16];      // row fragments (see Frag::row)
  uint32_t trans[D / 32][2];  // transposed fragments (see Frag::trans_frag)
  // Set up the row-fragment offsets and/or the transposed-fragment offsets (only what a
  // kernel reads, so no register is held for the other kind).
  template <bool ROWS, bool TRANS>
  __device__ __forceinline__ void init(const Frag<D>& fr) {
    if (ROWS) {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        rows[ks] = fr.rows[ks] + kBias;
        asm volatile("" : "+v"(rows[ks]));
      }
    }
    if (TRANS) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int hi = 0; hi < 2; ++hi) {
          trans[dt][hi] = fr.trans[dt][hi] + kBias;
          asm volatile("" : "+v"(trans[dt][hi]));
        }
    }
  }
  __device__ __forceinline__ bf16x8 row(const char* tile, int sub, int ks) const {
    return *reinterpret_cast<const bf16x8*>(tile + (rows[ks] - kBias) + sub * 32 * (D * 2));
  }
  // The same read with the tile's part of the address formed as one constant,
  // (tile - kBias + subtile offset), added to the biased register: the compiler then puts
  // it in the read's offset field instead of adding the tile address to an unbiased copy
  // of the register before every read.
  __device__ __forceinline__ bf16x8 row_folded(const char* tile, int sub, int ks) const {
    typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
    const uint32_t c = lds_addr(tile) + (uint32_t)(sub * 32 * (D * 2)) - kBias;
    return *reinterpret_cast<lds_bf16x8*>((uintptr_t)(rows[ks] + c));
  }
  __device__ __forceinline__ bf16x8 trans_frag(const char* tile, int sub, int h2, int dt) const {
    const int rb = (sub * 32 + 16 * h2) * (D * 2);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + (trans[dt][0] - kBias) + rb));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + (trans[dt][1] - kBias) + rb));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  }
};

// Empty volatile statement that takes two packed bf16 operands (and a float) as register
// inputs: it cannot move, so the instructions producing them stay before it.
__device__ __forceinline__ void pin_operands(const bf16x8 (&x)[2], float f) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 a = __builtin_bit_cast(u32x4, x[0]), b = __builtin_bit_cast(u32x4, x[1]);
  asm volatile("" ::"v"(a), "v"(b), "v"(f));
}

}  // namespace rr
