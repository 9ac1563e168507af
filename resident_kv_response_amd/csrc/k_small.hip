// HBM-bound kernels: softmax-statistics merge, backward preprocess D = rowsum(dO * O),
// ordered reduction of dQ partials, zero fill and the update-boundary axpy.
#include "k_common.h"
#include "kernels.h"

namespace rr {

// ---- merge ---------------------------------------------------------------------------
// Composition of softmax-statistics partials into the exact output
// (ai.thesatyajit.com/articles/longstraw-2m-rl, section "Two incompatible
// architectures, same transaction"): lse = ln sum_c e^{lse_c}, O = sum_c e^{lse_c-lse} O_c.
// Scalar form (any d_v or alignment): one wave per row, lane c reads lse_c once (lanes c,
// c + 64, ... for more parts), the wave reduces max and sum in a fixed order, and every
// lane then streams its column of all parts in part order, the weights broadcast from the
// lanes that hold them, several parts' loads in flight at once.
__global__ __launch_bounds__(256) void merge_kernel(int n_parts, int64_t rows, int d_v,
                                                    const float* __restrict__ part_o,
                                                    const float* __restrict__ part_lse,
                                                    float* __restrict__ o, float* __restrict__ lse,
                                                    bool use_geom, Geom g, int64_t ps, int64_t rs) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  bool pad = false;
  if (use_geom) {
    const int64_t kr = row / g.Hq;
    const int k = (int)(kr / g.R), r = (int)(kr % g.R);
    pad = r >= g.r_len[k];
  }
  float m = -INFINITY;
  const float* lrow = part_lse + row * rs;   // part c of this row at lrow[c * ps]
  if (!pad)
    for (int c = lane; c < n_parts; c += 64) m = fmaxf(m, lrow[(int64_t)c * ps]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  float out_lse = -INFINITY, inv = 0.0f;
  if (m != -INFINITY) {
    float den = 0.0f;
    for (int c = lane; c < n_parts; c += 64) den += expf(lrow[(int64_t)c * ps] - m);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off, 64);
    out_lse = m + logf(den);
    inv = 1.0f / den;
  }
  float* dst = o + row * d_v;
  // every lane runs every iteration (the weight broadcasts need all lanes); lanes past d_v
  // load and store nothing
  for (int base = 0; base < d_v; base += 64) {
    const int col = base + lane;
    const bool on = col < d_v;
    float acc = 0.0f;
    if (m != -INFINITY) {
      for (int c0 = 0; c0 < n_parts; c0 += 64) {
        // weights of parts c0 .. c0 + 63, one per lane (0 for -inf parts and past the end)
        const int cl = c0 + lane;
        const float lc = cl < n_parts ? lrow[(int64_t)cl * ps] : -INFINITY;
        const float wl = lc == -INFINITY ? 0.0f : expf(lc - m) * inv;
        const int n = min(64, n_parts - c0);
        int j = 0;
        for (; j + 4 <= n; j += 4) {          // four parts' loads in flight
          float x[4];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            x[u] = on ? part_o[((int64_t)(c0 + j + u) * ps + row * rs) * d_v + col] : 0.0f;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float w = __shfl(wl, j + u, 64);
            if (w != 0.0f) acc += w * x[u];
          }
        }
        for (; j < n; ++j) {
          const float w = __shfl(wl, j, 64);
          if (w != 0.0f && on) acc += w * part_o[((int64_t)(c0 + j) * ps + row * rs) * d_v + col];
        }
      }
    }
    if (on) dst[col] = acc;
  }
  if (lane == 0) lse[row] = out_lse;
}

// Two rows per wave for d_v % 4 == 0: lanes 0-31 merge one row, lanes 32-63 the next,
// each lane four consecutive columns of a 128-column pass.  The 32 lanes of a row reduce
// its lse_c (lane l holds parts l, l + 32, ...) in a fixed order, then stream the parts in
// part order with sixteen parts' loads in flight, the weight of part c broadcast from the
// lane that holds it.  Every lane of a 128-wide row is busy, where one wave per row left
// half of them idle at d_v = 128.
__global__ __launch_bounds__(256) void merge_rows_kernel(int n_parts, int64_t rows, int d_v,
                                                         const float* __restrict__ part_o,
                                                         const float* __restrict__ part_lse,
                                                         float* __restrict__ o, float* __restrict__ lse,
                                                         bool use_geom, Geom g, int64_t ps, int64_t rs) {
  const int l = threadIdx.x & 31;
  const int64_t row = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  if (row >= rows) return;   // whole 32-lane halves only: every shuffle below stays in its half
  bool pad = false;
  if (use_geom) {
    const int64_t kr = row / g.Hq;
    const int k = (int)(kr / g.R), r = (int)(kr % g.R);
    pad = r >= g.r_len[k];
  }
  float m = -INFINITY;
  const float* lrow = part_lse + row * rs;   // part c of this row at lrow[c * ps]
  if (!pad)
    for (int c = l; c < n_parts; c += 32) m = fmaxf(m, lrow[(int64_t)c * ps]);
#pragma unroll
  for (int off = 16; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 32));
  float out_lse = -INFINITY, inv = 0.0f;
  if (m != -INFINITY) {
    float den = 0.0f;
    for (int c = l; c < n_parts; c += 32) den += expf(lrow[(int64_t)c * ps] - m);
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) den += __shfl_xor(den, off, 32);
    out_lse = m + logf(den);
    inv = 1.0f / den;
  }
  float* dst = o + row * d_v;
  for (int base = 0; base < d_v; base += 128) {
    const int col = base + 4 * l;
    const bool on = col < d_v;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (m != -INFINITY) {
      const float* src0 = part_o + row * rs * d_v + col;
      const int64_t pstride = ps * d_v;
      for (int c0 = 0; c0 < n_parts; c0 += 32) {
        // weights of parts c0 .. c0 + 31, one per lane (0 for -inf parts and past the end)
        const int cl = c0 + l;
        const float lc = cl < n_parts ? lrow[(int64_t)cl * ps] : -INFINITY;
        const float wl = lc == -INFINITY ? 0.0f : expf(lc - m) * inv;
        const int n = min(32, n_parts - c0);
        int j = 0;
        for (; j + 16 <= n; j += 16) {          // sixteen parts' loads in flight
          float4 x[16];
#pragma unroll
          for (int u = 0; u < 16; ++u)
            x[u] = on ? *reinterpret_cast<const float4*>(src0 + (int64_t)(c0 + j + u) * pstride)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const float w = __shfl(wl, j + u, 32);
            if (w != 0.0f) {
              acc.x += w * x[u].x;
              acc.y += w * x[u].y;
              acc.z += w * x[u].z;
              acc.w += w * x[u].w;
            }
          }
        }
        for (; j < n; ++j) {
          const float w = __shfl(wl, j, 32);
          if (w != 0.0f && on) {
            const float4 x = *reinterpret_cast<const float4*>(src0 + (int64_t)(c0 + j) * pstride);
            acc.x += w * x.x;
            acc.y += w * x.y;
            acc.z += w * x.z;
            acc.w += w * x.w;
          }
        }
      }
    }
    if (on) *reinterpret_cast<float4*>(dst + col) = acc;
  }
  if (l == 0) lse[row] = out_lse;
}

hipError_t launch_merge(int n_parts, int64_t rows, int d_v, const float* part_o,
                        const float* part_lse, float* o, float* lse, const Geom* geom,
                        hipStream_t s) {
  if (rows == 0) return hipSuccess;
  Geom g{};
  if (geom) g = *geom;
  // the fused path's partials carry their layout in the geometry; rr_lse_merge's are part-major
  const int64_t ps = geom ? g.part_step : rows, rs = geom ? g.row_step : 1;
  const bool vec4 = (d_v % 4 == 0) && ((uintptr_t)part_o % 16 == 0) && ((uintptr_t)o % 16 == 0);
  if (vec4) {
    const int64_t blocks = (rows + 7) / 8;          // eight rows (half-waves) per workgroup
    hipLaunchKernelGGL(merge_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, n_parts, rows, d_v,
                       part_o, part_lse, o, lse, geom != nullptr, g, ps, rs);
  } else {
    const int64_t blocks = (rows + 3) / 4;          // four rows (waves) per workgroup
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(256), 0, s, n_parts, rows, d_v,
                       part_o, part_lse, o, lse, geom != nullptr, g, ps, rs);
  }
  return hipGetLastError();
}

// ---- D = rowsum(dO * O) ---------------------------------------------------------------
// 16 threads per (k, r, h) row, each reading 8 consecutive elements per step (one 16-byte
// load of bf16 dO, two of fp32 O); dO in its stored dtype.
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
    for (int d = 8 * lane16; d < g.dv; d += 128) {     // d_v is a multiple of 8
      const float4 o0 = *reinterpret_cast<const float4*>(orow + d);
      const float4 o1 = *reinterpret_cast<const float4*>(orow + d + 4);
      float x[8];
      if (BF16) {
        const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(d_o) + row * g.dv + d);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[2 * i] = __uint_as_float(w[i] << 16);
          x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
      } else {
        const float* src = static_cast<const float*>(d_o) + row * g.dv + d;
        const float4 a = *reinterpret_cast<const float4*>(src);
        const float4 b = *reinterpret_cast<const float4*>(src + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
      }
      const float y[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = fmaf(x[i], y[i], acc);
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
// dq = sum_c part_c in part order (deterministic); one float4 per thread.  The partials of
// row m (part c at row index c * part_step + m * row_step) are one contiguous run when
// they are row-major.
__global__ __launch_bounds__(256) void dq_reduce_kernel(Geom g, const float* __restrict__ part,
                                                        float* __restrict__ dq, int accumulate) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int q4 = g.dqk / 4;
  const int64_t per_k = (int64_t)(g.row_hi - g.row_lo) * g.Hq * q4;
  if (t >= per_k * g.K) return;
  const int k = (int)(t / per_k);
  const int64_t rem = t % per_k;
  const int r = g.row_lo + (int)(rem / ((int64_t)g.Hq * q4));
  const int hq4 = (int)(rem % ((int64_t)g.Hq * q4));
  const int64_t m = ((int64_t)k * g.R + r) * g.Hq + hq4 / q4;   // row index (k, r, h)
  const int col = (hq4 % q4) * 4;
  const int64_t off = m * g.dqk + col;
  const float* src = part + m * g.row_step * g.dqk + col;
  const int64_t pstep = g.part_step * g.dqk;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (r < g.r_len[k]) {
    for (int c = 0; c < g.n_parts; ++c) {
      const float4 x = *reinterpret_cast<const float4*>(src + c * pstep);
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
