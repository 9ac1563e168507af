// fp32 response-replay attention: one thread per query row (forward, dQ) or per
// (response key, 32-dim slice) (dK/dV), K/V tiles staged through LDS, fp32 arithmetic
// throughout with the accurate expf/logf.  Used for fp32 inputs; the bf16 path is the
// MFMA kernels.
//
// Rows are "flattened": for KV head g, index m = r * grp + hh enumerates response row r
// and query head h = g * grp + hh, so the grp query heads that read the same K/V run
// side by side.
#include "k_attn_tile.h"
#include "k_common.h"
#include "kernels.h"

namespace rr {

namespace {

constexpr int kF32Rows = 128;   // query rows per workgroup
constexpr int kF32Keys = 32;    // keys per LDS tile

struct PartRange {
  int64_t key0, key1;   // keys [key0, key1) of this part
  bool resp;            // response part: causal, keys index the response tensors
};

// Keys of part `part` for rows up to r_top (inclusive) of response k.
__device__ __forceinline__ PartRange part_range(const Geom& g, int part, int k, int r_top) {
  PartRange pr;
  if (part < g.n_chunks) {
    pr.key0 = (int64_t)part * g.chunk;
    pr.key1 = min(g.P, pr.key0 + g.chunk);
    pr.resp = false;
  } else {
    pr.key0 = 0;
    pr.key1 = g.resp_keys ? min(g.r_len[k], r_top + 1) : 0;
    pr.resp = true;
  }
  return pr;
}

}  // namespace

template <int D>
__global__ __launch_bounds__(kF32Rows) void fwd_partials_f32(Geom g, const float* __restrict__ q,
                                                             const float* __restrict__ k_p,
                                                             const float* __restrict__ v_p,
                                                             const float* __restrict__ k_r,
                                                             const float* __restrict__ v_r,
                                                             float* __restrict__ part_o,
                                                             float* __restrict__ part_lse) {
  __shared__ float ks[kF32Keys][D];
  __shared__ float vs[kF32Keys][D];
  const TileWork w = decode_tile_work(g, kF32Rows);
  if (!w.ok) return;
  const int m_hi = g.row_hi * g.grp;
  const int m = w.m0 + threadIdx.x;
  const int r = m / g.grp, hh = m % g.grp, h = w.g * g.grp + hh;
  const bool in_range = m < m_hi;
  const bool valid = in_range && r < g.r_len[w.k];
  const int r_top = min(m_hi - 1, w.m0 + kF32Rows - 1) / g.grp;
  const PartRange pr = part_range(g, w.part, w.k, r_top);

  float qv[D], o[D];
  const int64_t qrow = ((int64_t)w.k * g.R + r) * g.Hq + h;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qv[d] = valid ? q[qrow * D + d] : 0.0f;
    o[d] = 0.0f;
  }
  float mx = -INFINITY, l = 0.0f;
  const float* kb = pr.resp ? k_r + ((int64_t)w.k * g.R * g.Hkv + w.g) * D : k_p + (int64_t)w.g * D;
  const float* vb = pr.resp ? v_r + ((int64_t)w.k * g.R * g.Hkv + w.g) * D : v_p + (int64_t)w.g * D;
  const int64_t kstride = (int64_t)g.Hkv * D;
  for (int64_t t0 = pr.key0; t0 < pr.key1; t0 += kF32Keys) {
    __syncthreads();
    for (int e = threadIdx.x; e < kF32Keys * D; e += kF32Rows) {
      const int j = e / D, d = e % D;
      const int64_t key = t0 + j;
      ks[j][d] = key < pr.key1 ? kb[key * kstride + d] : 0.0f;
      vs[j][d] = key < pr.key1 ? vb[key * kstride + d] : 0.0f;
    }
    __syncthreads();
    const int nk = (int)min((int64_t)kF32Keys, pr.key1 - t0);
    for (int j = 0; j < nk; ++j) {
      if (pr.resp && t0 + j > r) break;
      float s = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) s += qv[d] * ks[j][d];
      s *= g.tau;
      if (s > mx) {
        const float alpha = expf(mx - s);   // 0 on the first visible key
        l = l * alpha + 1.0f;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] = o[d] * alpha + vs[j][d];
        mx = s;
      } else {
        const float p = expf(s - mx);
        l += p;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] += p * vs[j][d];
      }
    }
  }
  if (!in_range) return;
  const int64_t orow = (int64_t)w.part * g.part_step + (((int64_t)w.k * g.R + r) * g.Hq + h) * g.row_step;
  const bool live = valid && l > 0.0f;
  const float inv = live ? 1.0f / l : 0.0f;
#pragma unroll
  for (int d = 0; d < D; ++d) part_o[orow * D + d] = o[d] * inv;
  part_lse[orow] = live ? mx + logf(l) : -INFINITY;
}

template <int D>
__global__ __launch_bounds__(kF32Rows) void dq_partials_f32(Geom g, const float* __restrict__ q,
                                                            const float* __restrict__ k_p,
                                                            const float* __restrict__ v_p,
                                                            const float* __restrict__ k_r,
                                                            const float* __restrict__ v_r,
                                                            const float* __restrict__ d_o,
                                                            const float* __restrict__ lse,
                                                            const float* __restrict__ Dvec,
                                                            float* __restrict__ dq_part) {
  __shared__ float ks[kF32Keys][D];
  __shared__ float vs[kF32Keys][D];
  const TileWork w = decode_tile_work(g, kF32Rows);
  if (!w.ok) return;
  const int m_hi = g.row_hi * g.grp;
  const int m = w.m0 + threadIdx.x;
  const int r = m / g.grp, hh = m % g.grp, h = w.g * g.grp + hh;
  const bool in_range = m < m_hi;
  const bool valid = in_range && r < g.r_len[w.k];
  const int r_top = min(m_hi - 1, w.m0 + kF32Rows - 1) / g.grp;
  const PartRange pr = part_range(g, w.part, w.k, r_top);

  const int64_t qrow = ((int64_t)w.k * g.R + r) * g.Hq + h;
  float qv[D], dov[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qv[d] = valid ? q[qrow * D + d] : 0.0f;
    dov[d] = valid ? d_o[qrow * D + d] : 0.0f;
    acc[d] = 0.0f;
  }
  const float lrow = valid ? lse[qrow] : 0.0f;
  const float Drow = valid ? Dvec[qrow] : 0.0f;
  const float* kb = pr.resp ? k_r + ((int64_t)w.k * g.R * g.Hkv + w.g) * D : k_p + (int64_t)w.g * D;
  const float* vb = pr.resp ? v_r + ((int64_t)w.k * g.R * g.Hkv + w.g) * D : v_p + (int64_t)w.g * D;
  const int64_t kstride = (int64_t)g.Hkv * D;
  for (int64_t t0 = pr.key0; t0 < pr.key1; t0 += kF32Keys) {
    __syncthreads();
    for (int e = threadIdx.x; e < kF32Keys * D; e += kF32Rows) {
      const int j = e / D, d = e % D;
      const int64_t key = t0 + j;
      ks[j][d] = key < pr.key1 ? kb[key * kstride + d] : 0.0f;
      vs[j][d] = key < pr.key1 ? vb[key * kstride + d] : 0.0f;
    }
    __syncthreads();
    if (!valid) continue;
    const int nk = (int)min((int64_t)kF32Keys, pr.key1 - t0);
    for (int j = 0; j < nk; ++j) {
      if (pr.resp && t0 + j > r) break;
      float s = 0.0f, dp = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        s += qv[d] * ks[j][d];
        dp += dov[d] * vs[j][d];
      }
      const float p = expf(s * g.tau - lrow);
      const float ds = p * (dp - Drow);
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] += ds * ks[j][d];
    }
  }
  if (!in_range) return;
  const int64_t orow = (int64_t)w.part * g.part_step + (((int64_t)w.k * g.R + r) * g.Hq + h) * g.row_step;
#pragma unroll
  for (int d = 0; d < D; ++d) dq_part[orow * D + d] = valid ? acc[d] * g.tau : 0.0f;
}

// dK/dV of response keys: one workgroup per (k, g, 32 keys); thread = (key, 32-dim slice).
// Loops over the query rows [row_lo, row_hi) that see the key (r >= key) and every query
// head of the group; adds into dk_r/dv_r.
template <int D>
__global__ __launch_bounds__(32 * (D / 32)) void dkdv_f32(Geom g, int key_hi,
                                                          const float* __restrict__ q,
                                                          const float* __restrict__ k_r,
                                                          const float* __restrict__ v_r,
                                                          const float* __restrict__ d_o,
                                                          const float* __restrict__ lse,
                                                          const float* __restrict__ Dvec,
                                                          float* __restrict__ dk_r,
                                                          float* __restrict__ dv_r) {
  constexpr int SL = D / 32;    // slices per key
  __shared__ float ks[32][D];
  __shared__ float vs[32][D];
  const int n_kt = (key_hi + 31) / 32;
  const int64_t n_work = (int64_t)g.K * g.Hkv * n_kt;
  const int64_t idx = blockIdx.x;
  if (idx >= n_work) return;
  const int kt = (int)(idx % n_kt);
  const int gh = (int)((idx / n_kt) % g.Hkv);
  const int k = (int)(idx / ((int64_t)n_kt * g.Hkv));
  const int jl = threadIdx.x / SL, sl = threadIdx.x % SL;
  const int j = kt * 32 + jl;
  const int kend = min(key_hi, g.r_len[k]);
  const int64_t kvrow = ((int64_t)k * g.R + j) * g.Hkv + gh;
  for (int e = threadIdx.x; e < 32 * D; e += 32 * SL) {
    const int jj = e / D, d = e % D;
    const int key = kt * 32 + jj;
    const int64_t rowoff = (((int64_t)k * g.R + key) * g.Hkv + gh) * D + d;
    ks[jj][d] = key < kend ? k_r[rowoff] : 0.0f;
    vs[jj][d] = key < kend ? v_r[rowoff] : 0.0f;
  }
  __syncthreads();
  if (j >= kend) return;
  float dk[32], dv[32];
#pragma unroll
  for (int t = 0; t < 32; ++t) dk[t] = dv[t] = 0.0f;
  const int r_end = min(g.row_hi, g.r_len[k]);
  for (int r = max(g.row_lo, j); r < r_end; ++r) {
    for (int hh = 0; hh < g.grp; ++hh) {
      const int64_t qrow = ((int64_t)k * g.R + r) * g.Hq + gh * g.grp + hh;
      const float* qp = q + qrow * D;
      const float* dop = d_o + qrow * D;
      float s = 0.0f, dp = 0.0f;
      for (int d = 0; d < D; ++d) {
        s += qp[d] * ks[jl][d];
        dp += dop[d] * vs[jl][d];
      }
      const float p = expf(s * g.tau - lse[qrow]);
      const float ds = p * (dp - Dvec[qrow]);
#pragma unroll
      for (int t = 0; t < 32; ++t) {
        dk[t] += ds * qp[sl * 32 + t];
        dv[t] += p * dop[sl * 32 + t];
      }
    }
  }
#pragma unroll
  for (int t = 0; t < 32; ++t) {
    dk_r[kvrow * D + sl * 32 + t] += dk[t] * g.tau;
    dv_r[kvrow * D + sl * 32 + t] += dv[t];
  }
}

namespace {

// The forward and dQ kernels share the bf16 kernels' work order (decode_tile_work), with
// one workgroup per kF32Rows flattened rows.
int64_t row_work(const Geom& g, int rows_per_wg) { return tile_work_count(g, rows_per_wg); }

}  // namespace

hipError_t launch_fwd_partials_f32(const Geom& g, const AttnPtrs& a, hipStream_t s) {
  const int64_t n = row_work(g, kF32Rows);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)xcd_grid(n)), block(kF32Rows);
  const float *q = (const float*)a.q, *kp = (const float*)a.k_p, *vp = (const float*)a.v_p;
  const float *kr = (const float*)a.k_r, *vr = (const float*)a.v_r;
  if (g.dqk == 64)
    hipLaunchKernelGGL(fwd_partials_f32<64>, grid, block, 0, s, g, q, kp, vp, kr, vr, a.part_o, a.part_lse);
  else
    hipLaunchKernelGGL(fwd_partials_f32<128>, grid, block, 0, s, g, q, kp, vp, kr, vr, a.part_o, a.part_lse);
  return hipGetLastError();
}

hipError_t launch_dq_partials_f32(const Geom& g, const AttnPtrs& a, hipStream_t s) {
  const int64_t n = row_work(g, kF32Rows);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)xcd_grid(n)), block(kF32Rows);
  const float *q = (const float*)a.q, *kp = (const float*)a.k_p, *vp = (const float*)a.v_p;
  const float *kr = (const float*)a.k_r, *vr = (const float*)a.v_r, *dO = (const float*)a.d_o;
  if (g.dqk == 64)
    hipLaunchKernelGGL(dq_partials_f32<64>, grid, block, 0, s, g, q, kp, vp, kr, vr, dO, a.lse, a.Dvec,
                       a.dq_part);
  else
    hipLaunchKernelGGL(dq_partials_f32<128>, grid, block, 0, s, g, q, kp, vp, kr, vr, dO, a.lse, a.Dvec,
                       a.dq_part);
  return hipGetLastError();
}

hipError_t launch_dkdv_f32(const Geom& g, const AttnPtrs& a, int key_hi, hipStream_t s) {
  if (key_hi <= 0) return hipSuccess;
  const int n_kt = (key_hi + 31) / 32;
  const int64_t n = (int64_t)g.K * g.Hkv * n_kt;
  const float *q = (const float*)a.q, *kr = (const float*)a.k_r, *vr = (const float*)a.v_r;
  const float* dO = (const float*)a.d_o;
  if (g.dqk == 64)
    hipLaunchKernelGGL(dkdv_f32<64>, dim3((unsigned)n), dim3(64), 0, s, g, key_hi, q, kr, vr, dO, a.lse,
                       a.Dvec, a.dk_r, a.dv_r);
  else
    hipLaunchKernelGGL(dkdv_f32<128>, dim3((unsigned)n), dim3(128), 0, s, g, key_hi, q, kr, vr, dO, a.lse,
                       a.Dvec, a.dk_r, a.dv_r);
  return hipGetLastError();
}

}  // namespace rr
