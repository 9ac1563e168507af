// HBM-bound kernels: softmax-statistics merge, backward preprocess D = rowsum(dO * O),
// ordered reduction of dQ partials, zero fill and the update-boundary axpy.
#include "k_common.h"
#include "kernels.h"

namespace rr {

// ---- merge ---------------------------------------------------------------------------
// Composition of softmax-statistics partials into the exact output
// (ai.thesatyajit.com/articles/longstraw-2m-rl, section "Two incompatible
// architectures, same transaction"): lse = ln sum_c e^{lse_c}, O = sum_c e^{lse_c-lse} O_c.
// One thread owns VEC consecutive output elements of one row; the n_parts statistics of
// the row are re-read from L1/L2 by each of its threads (tiny next to the O_c traffic).
template <int VEC>
__global__ __launch_bounds__(256) void merge_kernel(int n_parts, int64_t rows, int d_v,
                                                    const float* __restrict__ part_o,
                                                    const float* __restrict__ part_lse,
                                                    float* __restrict__ o, float* __restrict__ lse,
                                                    bool use_geom, Geom g) {
  const int tpr = (d_v + VEC - 1) / VEC;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = t / tpr;
  const int col = (int)(t % tpr) * VEC;
  if (row >= rows) return;
  bool pad = false;
  if (use_geom) {
    const int64_t kr = row / g.Hq;
    const int k = (int)(kr / g.R), r = (int)(kr % g.R);
    pad = r >= g.r_len[k];
  }
  float m = -INFINITY;
  if (!pad)
    for (int c = 0; c < n_parts; ++c) m = fmaxf(m, part_lse[(int64_t)c * rows + row]);
  float acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.0f;
  float out_lse = -INFINITY;
  if (m != -INFINITY) {
    float den = 0.0f;
    for (int c = 0; c < n_parts; ++c) den += expf(part_lse[(int64_t)c * rows + row] - m);
    out_lse = m + logf(den);
    for (int c = 0; c < n_parts; ++c) {
      const float lc = part_lse[(int64_t)c * rows + row];
      if (lc == -INFINITY) continue;
      const float w = expf(lc - out_lse);
      const float* src = part_o + ((int64_t)c * rows + row) * d_v + col;
      if constexpr (VEC == 4) {
        const float4 x = *reinterpret_cast<const float4*>(src);
        acc[0] += w * x.x;
        acc[1] += w * x.y;
        acc[2] += w * x.z;
        acc[3] += w * x.w;
      } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v)
          if (col + v < d_v) acc[v] += w * src[v];
      }
    }
  }
  float* dst = o + row * d_v + col;
  if constexpr (VEC == 4) {
    *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  } else {
#pragma unroll
    for (int v = 0; v < VEC; ++v)
      if (col + v < d_v) dst[v] = acc[v];
  }
  if (col == 0) lse[row] = out_lse;
}

hipError_t launch_merge(int n_parts, int64_t rows, int d_v, const float* part_o,
                        const float* part_lse, float* o, float* lse, const Geom* geom,
                        hipStream_t s) {
  if (rows == 0) return hipSuccess;
  Geom g{};
  if (geom) g = *geom;
  const bool vec4 = (d_v % 4 == 0) && ((uintptr_t)part_o % 16 == 0) && ((uintptr_t)o % 16 == 0);
  const int vec = vec4 ? 4 : 1;
  const int64_t threads = rows * ((d_v + vec - 1) / vec);
  const int64_t blocks = (threads + 255) / 256;
  if (vec4)
    hipLaunchKernelGGL(merge_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, s, n_parts, rows, d_v,
                       part_o, part_lse, o, lse, geom != nullptr, g);
  else
    hipLaunchKernelGGL(merge_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, s, n_parts, rows, d_v,
                       part_o, part_lse, o, lse, geom != nullptr, g);
  return hipGetLastError();
}

// ---- D = rowsum(dO * O) ---------------------------------------------------------------
// 16 threads per (k, r, h) row; dO in its stored dtype, O in fp32.
template <bool BF16>
__global__ __launch_bounds__(256) void bwd_pre_kernel(Geom g, const float* __restrict__ o,
                                                      const void* __restrict__ d_o,
                                                      float* __restrict__ Dvec) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int lane16 = threadIdx.x & 15;
  const int64_t rows_per_k = (int64_t)(g.row_hi - g.row_lo) * g.Hq;
  const int64_t idx = t >> 4;
  if (idx >= rows_per_k * g.K) return;
  const int k = (int)(idx / rows_per_k);
  const int64_t rem = idx % rows_per_k;
  const int r = g.row_lo + (int)(rem / g.Hq);
  const int h = (int)(rem % g.Hq);
  const int64_t row = ((int64_t)k * g.R + r) * g.Hq + h;
  float acc = 0.0f;
  if (r < g.r_len[k]) {
    const float* orow = o + row * g.dv;
    for (int d = lane16; d < g.dv; d += 16) {
      float x;
      if (BF16)
        x = bf16_bits_to_f32(static_cast<const uint16_t*>(d_o)[row * g.dv + d]);
      else
        x = static_cast<const float*>(d_o)[row * g.dv + d];
      acc += x * orow[d];
    }
  }
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 16);
  if (lane16 == 0) Dvec[row] = acc;
}

hipError_t launch_bwd_pre(const Geom& g, int dtype, const float* o, const void* d_o, float* Dvec,
                          hipStream_t s) {
  const int64_t rows = (int64_t)g.K * (g.row_hi - g.row_lo) * g.Hq;
  if (rows == 0) return hipSuccess;
  const int64_t blocks = (rows * 16 + 255) / 256;
  if (dtype == RR_BF16)
    hipLaunchKernelGGL(bwd_pre_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, g, o, d_o, Dvec);
  else
    hipLaunchKernelGGL(bwd_pre_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, g, o, d_o, Dvec);
  return hipGetLastError();
}

// ---- ordered dQ reduction ------------------------------------------------------------
// dq = sum_c part_c in part order (deterministic); one float4 per thread.
__global__ __launch_bounds__(256) void dq_reduce_kernel(Geom g, const float* __restrict__ part,
                                                        float* __restrict__ dq, int accumulate) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int q4 = g.dqk / 4;
  const int64_t per_k = (int64_t)(g.row_hi - g.row_lo) * g.Hq * q4;
  if (t >= per_k * g.K) return;
  const int k = (int)(t / per_k);
  const int64_t rem = t % per_k;
  const int r = g.row_lo + (int)(rem / ((int64_t)g.Hq * q4));
  const int64_t off = (((int64_t)k * g.R + r) * g.Hq) * g.dqk + (rem % ((int64_t)g.Hq * q4)) * 4;
  const int64_t stride = (int64_t)g.K * g.R * g.Hq * g.dqk;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (r < g.r_len[k]) {
    for (int c = 0; c < g.n_parts; ++c) {
      const float4 x = *reinterpret_cast<const float4*>(part + c * stride + off);
      acc.x += x.x;
      acc.y += x.y;
      acc.z += x.z;
      acc.w += x.w;
    }
  }
  float4* dst = reinterpret_cast<float4*>(dq + off);
  if (accumulate) {
    const float4 y = *dst;
    acc.x += y.x;
    acc.y += y.y;
    acc.z += y.z;
    acc.w += y.w;
  }
  *dst = acc;
}

hipError_t launch_dq_reduce(const Geom& g, const float* dq_part, float* dq, int accumulate,
                            hipStream_t s) {
  const int64_t n = (int64_t)g.K * (g.row_hi - g.row_lo) * g.Hq * (g.dqk / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(dq_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, g,
                     dq_part, dq, accumulate);
  return hipGetLastError();
}

// ---- zero fill of a row range -----------------------------------------------------------
__global__ __launch_bounds__(256) void zero_rows_kernel(float* __restrict__ x, int R, int lo,
                                                        int hi, int64_t row_elems, int64_t per_k,
                                                        int64_t n) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  const int64_t k = t / per_k;
  const int64_t e = t % per_k;
  x[(k * R + lo) * row_elems + e] = 0.0f;
}

hipError_t launch_zero_rows(float* x, int K, int R, int lo, int hi, int64_t row_elems,
                            hipStream_t s) {
  if (hi <= lo) return hipSuccess;
  const int64_t per_k = (int64_t)(hi - lo) * row_elems;
  const int64_t n = per_k * K;
  hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, R, lo,
                     hi, row_elems, per_k, n);
  return hipGetLastError();
}

// ---- update-boundary accumulation -----------------------------------------------------
__global__ __launch_bounds__(256) void axpy_kernel(float* __restrict__ acc,
                                                   const float* __restrict__ g, int64_t n,
                                                   float scale) {
  const int64_t i4 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i4 + 3 < n) {
    const float4 x = *reinterpret_cast<const float4*>(g + i4);
    float4 y = *reinterpret_cast<float4*>(acc + i4);
    y.x += scale * x.x;
    y.y += scale * x.y;
    y.z += scale * x.z;
    y.w += scale * x.w;
    *reinterpret_cast<float4*>(acc + i4) = y;
  } else {
    for (int64_t i = i4; i < n; ++i) acc[i] += scale * g[i];
  }
}

__global__ __launch_bounds__(256) void axpy_scalar_kernel(float* __restrict__ acc,
                                                          const float* __restrict__ g, int64_t n,
                                                          float scale) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) acc[i] += scale * g[i];
}

hipError_t launch_axpy(float* acc, const float* g, int64_t n, float scale, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if ((uintptr_t)acc % 16 == 0 && (uintptr_t)g % 16 == 0) {
    const int64_t th = (n + 3) / 4;
    hipLaunchKernelGGL(axpy_kernel, dim3((unsigned)((th + 255) / 256)), dim3(256), 0, s, acc, g, n, scale);
  } else {
    hipLaunchKernelGGL(axpy_scalar_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, acc, g,
                       n, scale);
  }
  return hipGetLastError();
}

}  // namespace rr
