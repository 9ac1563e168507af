// Device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rr_internal.h"

namespace rr {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Finite stand-in for "no key seen yet" so that differences never form inf - inf.
constexpr float kNegBig = -1.0e30f;

// Exact bf16 -> fp32 widening of a stored bit pattern.
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// Round-to-nearest-even fp32 pair -> packed bf16x2: one v_cvt_pk_bf16_f32 on gfx950.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Sum of the 8 bf16 values of two packed MFMA operands (x + (lo + hi) per pair, fp32),
// by v_dot2c_f32_bf16 against (1, 1): half the instructions of 16 fp32 adds, and the sum
// is that of exactly the rounded values the MFMA consumes.
__device__ __forceinline__ float sum_bf16x8(uint4 u, float x) {
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
  x = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, u.x), one, x, false);
  x = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, u.y), one, x, false);
  x = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, u.z), one, x, false);
  x = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, u.w), one, x, false);
  return x;
}

// Wave priority around matrix-core blocks: with two waves per SIMD, the wave that has
// MFMAs to issue goes first, and the other wave's vector work fills the matrix core's
// busy cycles.  The scheduling barriers keep the compiler from moving instructions
// across the priority changes.
__device__ __forceinline__ void prio_mfma() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(1);
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void prio_valu() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
}

// 16-byte vector <-> 8 bf16 MFMA operand.
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup -> work-item map that keeps consecutive work items on one XCD.  Workgroups
// are dispatched round-robin over the 8 XCDs (blockIdx % 8), each XCD with its own L2;
// work items that read the same K/V chunk are numbered consecutively, so giving XCD x
// the contiguous range [x*per, (x+1)*per) makes the workgroups resident on one XCD
// stream the same chunk and share it through that XCD's L2.  Launch 8*per workgroups;
// returns -1 for the padding workgroups beyond n_work.
__device__ __forceinline__ int64_t xcd_work_index(int64_t n_work) {
  const int64_t per = (n_work + 7) / 8;
  const int64_t b = blockIdx.x;
  const int64_t w = (b % 8) * per + b / 8;
  return w < n_work ? w : -1;
}

inline int64_t xcd_grid(int64_t n_work) { return ((n_work + 7) / 8) * 8; }

}  // namespace rr
