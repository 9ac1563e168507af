// bf16 forward partials on MFMA (gfx950).
//
// One workgroup = one (response k, KV head g, part, 256-row tile).  A part is one prompt
// chunk [c*chunk, (c+1)*chunk) or the response's own causal keys; each part keeps its own
// softmax statistics (running max m, running sum l) and writes O_c = O~_c / l and
// lse_c = m + ln l, which are then composed exactly (ai.thesatyajit.com/articles/
// longstraw-2m-rl, section "Two incompatible architectures, same transaction").
//
// Rows: flattened m = r * grp + hh over the grp query heads that read KV head g, so one
// K/V tile feeds grp heads.  4 waves x 64 rows; each wave keeps its Q fragments and its
// O^T accumulators (d x rows, fp32) in registers for the whole part.
//
// Per 64-key stage: K as [key][d] and V transposed as [d][key] in LDS (double-buffered;
// the next stage's global loads are issued before the current stage's MFMAs).  Per
// 32-key subtile and 32-row N-tile:  S^T = K Q^T (D/16 MFMAs), base-2 online softmax with
// a lazy rescale (the reference maximum only moves when a row's maximum grows by more
// than 2^8, keeping every p <= 256), P^T rounded to bf16, O^T += V^T P^T (D/16 MFMAs).
#include "k_attn_tile.h"
#include "kernels.h"

namespace rr {

constexpr float kRescaleThreshold = 8.0f;   // log2 of the largest p between rescales

template <int D>
__global__ __launch_bounds__(256, 1) void fwd_partials_bf16(
    Geom g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_p,
    const uint16_t* __restrict__ v_p, const uint16_t* __restrict__ k_r,
    const uint16_t* __restrict__ v_r, float* __restrict__ part_o, float* __restrict__ part_lse) {
  using C = TileCfg<D>;
  constexpr int STAGE = C::NORM_ELEMS + C::TRANS_ELEMS;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];

  const TileWork w = decode_tile_work(g, C::BM);
  if (!w.ok) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hl = lane >> 5, col = lane & 31;
  const int m_hi = g.row_hi * g.grp;
  const int r_first = w.m0 / g.grp;
  const int r_top = (min(m_hi, w.m0 + C::BM) - 1) / g.grp;
  const int rl = g.r_len[w.k];

  // keys of this part
  const bool resp = w.part >= g.n_chunks;
  int64_t key0, key1;
  if (!resp) {
    key0 = (int64_t)w.part * g.chunk;
    key1 = min(g.P, key0 + g.chunk);
  } else {
    key0 = 0;
    key1 = min(rl, r_top + 1);
  }
  const int64_t stride = (int64_t)g.Hkv * D;
  const uint16_t* kb = resp ? k_r + ((int64_t)w.k * g.R * g.Hkv + w.g) * D : k_p + (int64_t)w.g * D;
  const uint16_t* vb = resp ? v_r + ((int64_t)w.k * g.R * g.Hkv + w.g) * D : v_p + (int64_t)w.g * D;
  const int n_keys = (r_first >= rl) ? 0 : (int)(key1 - key0);
  const int n_tiles = (n_keys + C::BN - 1) / C::BN;

  // this lane's rows: visibility limit (relative key index) and Q fragments
  int lim[C::NT];
  bool valid[C::NT];
  int64_t orow[C::NT];
  bf16x8 qf[C::NT][C::KS];
#pragma unroll
  for (int t = 0; t < C::NT; ++t) {
    const int m = w.m0 + wave * C::ROWS_W + t * 32 + col;
    const int r = m / g.grp, h = w.g * g.grp + m % g.grp;
    valid[t] = m < m_hi && r < rl;
    lim[t] = resp ? min(r, n_keys - 1) : n_keys - 1;
    orow[t] = m < m_hi ? (((int64_t)w.part * g.K + w.k) * g.R + r) * g.Hq + h : -1;
    const uint16_t* qrow = q + (((int64_t)w.k * g.R + r) * g.Hq + h) * D;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      qf[t][ks] = as_bf16x8(valid[t] ? *reinterpret_cast<const uint4*>(qrow + ks * 16 + hl * 8)
                                     : make_uint4(0, 0, 0, 0));
  }
  int wmin = min(lim[0], lim[C::NT - 1]), wmax = max(lim[0], lim[C::NT - 1]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    wmin = min(wmin, __shfl_xor(wmin, off, 64));
    wmax = max(wmax, __shfl_xor(wmax, off, 64));
  }

  f32x16 acc[C::NT][C::DT];
  float m_run[C::NT], l_run[C::NT];
#pragma unroll
  for (int t = 0; t < C::NT; ++t) {
    m_run[t] = kNegBig;
    l_run[t] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[t][dt][i] = 0.0f;
  }

  RowPieces<D, C::PIECES_PER_THREAD> kreg;
  QuadPieces<D, C::QUADS_PER_THREAD> vreg;
  if (n_tiles > 0) {
    load_pieces<D>(kreg, kb, key0, key0 + n_keys, stride);
    load_quads<D>(vreg, vb, key0, key0 + n_keys, stride);
    store_pieces<D>(kreg, lds);
    store_quads_transposed<D>(vreg, lds + C::NORM_ELEMS);
  }
  __syncthreads();

  for (int it = 0; it < n_tiles; ++it) {
    if (it + 1 < n_tiles) {
      const int64_t nk0 = key0 + (int64_t)(it + 1) * C::BN;
      load_pieces<D>(kreg, kb, nk0, key0 + n_keys, stride);
      load_quads<D>(vreg, vb, nk0, key0 + n_keys, stride);
    }
    const uint16_t* Ks = lds + (it & 1) * STAGE;
    const uint16_t* Vt = Ks + C::NORM_ELEMS;
#pragma unroll
    for (int sub = 0; sub < C::BN / 32; ++sub) {
      const int rel = it * C::BN + sub * 32;
      if (rel > wmax) continue;            // every row of this wave is past its last key
      f32x16 s[C::NT];
#pragma unroll
      for (int t = 0; t < C::NT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[t][i] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bf16x8 a =
            as_bf16x8(*reinterpret_cast<const uint4*>(Ks + (sub * 32 + col) * C::ROW + ks * 16 + hl * 8));
#pragma unroll
        for (int t = 0; t < C::NT; ++t) s[t] = mfma32x32x16(a, qf[t][ks], s[t]);
      }
      const bool need_mask = rel + 31 > wmin;
      bool grow = false;
      float m_new[C::NT];
#pragma unroll
      for (int t = 0; t < C::NT; ++t) {
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float x = s[t][i] * g.c2;
          if (need_mask) {
            const int key = rel + (i >> 2) * 8 + hl * 4 + (i & 3);
            if (key > lim[t]) x = -INFINITY;
          }
          s[t][i] = x;
          mx = fmaxf(mx, x);
        }
        mx = fmaxf(mx, partner32(mx));
        m_new[t] = fmaxf(m_run[t], mx);
        grow |= m_new[t] > m_run[t] + kRescaleThreshold;
      }
      if (__any(grow)) {
#pragma unroll
        for (int t = 0; t < C::NT; ++t) {
          const float alpha = fast_exp2(m_run[t] - m_new[t]);
          l_run[t] *= alpha;
#pragma unroll
          for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[t][dt][i] *= alpha;
          m_run[t] = m_new[t];
        }
      }
      bf16x8 pf[C::NT][2];
#pragma unroll
      for (int t = 0; t < C::NT; ++t) {
        float p[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          p[i] = fast_exp2(s[t][i] - m_run[t]);
          l_run[t] += p[i];
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          uint4 u;
          u.x = pack_bf16x2(p[8 * h2 + 0], p[8 * h2 + 1]);
          u.y = pack_bf16x2(p[8 * h2 + 2], p[8 * h2 + 3]);
          u.z = pack_bf16x2(p[8 * h2 + 4], p[8 * h2 + 5]);
          u.w = pack_bf16x2(p[8 * h2 + 6], p[8 * h2 + 7]);
          pf[t][h2] = as_bf16x8(u);
        }
      }
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const bf16x8 a = as_bf16x8(
              *reinterpret_cast<const uint4*>(Vt + (dt * 32 + col) * C::TROW + sub * 32 + h2 * 16 + hl * 8));
#pragma unroll
          for (int t = 0; t < C::NT; ++t) acc[t][dt] = mfma32x32x16(a, pf[t][h2], acc[t][dt]);
        }
      }
    }
    if (it + 1 < n_tiles) {
      uint16_t* nxt = lds + ((it + 1) & 1) * STAGE;
      store_pieces<D>(kreg, nxt);
      store_quads_transposed<D>(vreg, nxt + C::NORM_ELEMS);
    }
    __syncthreads();
  }

#pragma unroll
  for (int t = 0; t < C::NT; ++t) {
    const float l = l_run[t] + partner32(l_run[t]);
    if (orow[t] < 0) continue;
    const bool live = valid[t] && l > 0.0f;
    const float inv = live ? 1.0f / l : 0.0f;
    float* dst = part_o + orow[t] * D;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d0 = dt * 32 + i4 * 8 + hl * 4;
        *reinterpret_cast<float4*>(dst + d0) =
            make_float4(acc[t][dt][4 * i4 + 0] * inv, acc[t][dt][4 * i4 + 1] * inv,
                        acc[t][dt][4 * i4 + 2] * inv, acc[t][dt][4 * i4 + 3] * inv);
      }
    if (hl == 0) part_lse[orow[t]] = live ? (m_run[t] + log2f(l)) * kLn2 : -INFINITY;
  }
}

hipError_t launch_fwd_partials_bf16(const Geom& g, const AttnPtrs& a, hipStream_t s) {
  const int64_t n = tile_work_count(g, TileCfg<128>::BM);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)xcd_grid(n)), block(256);
  const uint16_t *q = (const uint16_t*)a.q, *kp = (const uint16_t*)a.k_p, *vp = (const uint16_t*)a.v_p;
  const uint16_t *kr = (const uint16_t*)a.k_r, *vr = (const uint16_t*)a.v_r;
  if (g.dqk == 64)
    hipLaunchKernelGGL(fwd_partials_bf16<64>, grid, block, 0, s, g, q, kp, vp, kr, vr, a.part_o, a.part_lse);
  else
    hipLaunchKernelGGL(fwd_partials_bf16<128>, grid, block, 0, s, g, q, kp, vp, kr, vr, a.part_o, a.part_lse);
  return hipGetLastError();
}

}  // namespace rr
