// bf16 response dK/dV on MFMA (gfx950): the reverse block walk over the response's own
// keys.
//
// Source of the contract: ai.thesatyajit.com/articles/longstraw-2m-rl, sections "The
// move: change the graph boundary" (the resident prompt state is a stop-gradient: only
// the direct response gradient is formed) and "Two incompatible architectures, same
// transaction" (response blocks replayed in reverse; K/V gradient storage only for
// what a response backward touches).  No kernel here reads or writes a prompt gradient.
//
// dkdv_bf16: key-parallel over the response keys, one workgroup per (k, g, 128 keys),
// each wave owning 32 keys (K, V fragments in registers, dK^T and dV^T accumulators in
// registers).  The workgroup walks the query rows of one response block in 32-row tiles
// staged in LDS (plain and transposed), computing S = Q K^T and dP = dO V^T per tile and
// dV^T += dO^T P, dK^T += Q^T dS, then adds its result into dk_r / dv_r.  Launched once
// per block, last block first.
#include "k_attn_tile.h"
#include "k_lds.h"
#include "kernels.h"

namespace rr {

// ---- response dK / dV --------------------------------------------------------------------

template <int D>
struct KvCfg {
  static constexpr int WAVES = 4;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int KEYS = 32 * WAVES;        // response keys per workgroup
  static constexpr int QT = 32;                  // flattened query rows per LDS stage
  static constexpr int KS = D / 16, DT = D / 32;
  static constexpr int ROW = D + 8;              // [row][d]
  static constexpr int TROW = QT + 8;            // [d][row]
  static constexpr int PLAIN = QT * ROW;
  static constexpr int TRANS = D * TROW;
  static constexpr int QUADS = (QT / 4) * (D / 8);            // per tensor
  static constexpr int STAGE_U16 = 2 * PLAIN + 2 * TRANS;    // Qs, dOs, Qt, dOt
  static constexpr int STAGE_F32 = 3 * QT;                   // lse2, D, row index
};

template <int D>
__global__ __launch_bounds__(256, 1) void dkdv_bf16(
    Geom g, int key_hi, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_r,
    const uint16_t* __restrict__ v_r, const uint16_t* __restrict__ d_o,
    const float* __restrict__ lse, const float* __restrict__ Dvec, float* __restrict__ dk_r,
    float* __restrict__ dv_r) {
  using C = KvCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t lds_u16[2 * C::STAGE_U16];
  __shared__ __attribute__((aligned(16))) float lds_f32[2 * C::STAGE_F32];

  const int n_kt = (key_hi + C::KEYS - 1) / C::KEYS;
  const int64_t idx = xcd_work_index((int64_t)g.K * g.Hkv * n_kt);
  if (idx < 0) return;
  const int kt = (int)(idx % n_kt);
  const int gh = (int)((idx / n_kt) % g.Hkv);
  const int k = (int)(idx / ((int64_t)n_kt * g.Hkv));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hl = lane >> 5, col = lane & 31;
  const int rl = g.r_len[k];
  const int key_end = min(key_hi, rl);
  const int j0 = kt * C::KEYS;
  if (j0 >= key_end) return;
  const int j0w = j0 + wave * 32;
  const int my_key = j0w + col;

  // this wave's K and V fragments (B operands): key my_key, dims 16ks + 8hl .. +8
  bf16x8 kf[C::KS], vf[C::KS];
  const int64_t kvrow = ((int64_t)k * g.R + my_key) * g.Hkv + gh;
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const bool ok = my_key < key_end;
    kf[ks] = as_bf16x8(ok ? *reinterpret_cast<const uint4*>(k_r + kvrow * D + ks * 16 + hl * 8)
                          : make_uint4(0, 0, 0, 0));
    vf[ks] = as_bf16x8(ok ? *reinterpret_cast<const uint4*>(v_r + kvrow * D + ks * 16 + hl * 8)
                          : make_uint4(0, 0, 0, 0));
  }

  // query rows (flattened m = r * grp + hh) that can see any key of this workgroup
  const int r_lo = max(g.row_lo, j0), r_hi = min(g.row_hi, rl);
  const int mq_lo = r_lo * g.grp, mq_hi = r_hi * g.grp;
  const int n_qt = mq_hi > mq_lo ? (mq_hi - mq_lo + C::QT - 1) / C::QT : 0;

  f32x16 dk[C::DT], dv[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) dk[dt][i] = dv[dt][i] = 0.0f;

  // staging: quad p < QUADS -> Q, else dO; rows 4*rq .. 4*rq+3 of the tile, dims col8..+8
  uint4 st[4];
  float st_l = 0.0f, st_d = 0.0f;
  int st_r = 0;
  auto load_stage = [&](int mt) {
    const int p = threadIdx.x;
    if (p < 2 * C::QUADS) {
      const bool is_q = p < C::QUADS;
      const int pp = is_q ? p : p - C::QUADS;
      const int rq = pp / (D / 8), c8 = (pp % (D / 8)) * 8;
      const uint16_t* src = is_q ? q : d_o;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int m = mt + 4 * rq + u;
        if (m < mq_hi) {
          const int r = m / g.grp, h = gh * g.grp + m % g.grp;
          st[u] = *reinterpret_cast<const uint4*>(src + (((int64_t)k * g.R + r) * g.Hq + h) * D + c8);
        } else {
          st[u] = make_uint4(0, 0, 0, 0);
        }
      }
    }
    if (threadIdx.x < C::QT) {
      const int m = mt + threadIdx.x;
      if (m < mq_hi) {
        const int r = m / g.grp, h = gh * g.grp + m % g.grp;
        const int64_t row = ((int64_t)k * g.R + r) * g.Hq + h;
        st_l = lse[row] * kLog2e;
        st_d = Dvec[row];
        st_r = r;
      } else {
        st_l = INFINITY;   // p = 0
        st_d = 0.0f;
        st_r = 0x7fffffff;
      }
    }
  };
  auto store_stage = [&](int buf) {
    uint16_t* base = lds_u16 + buf * C::STAGE_U16;
    float* fb = lds_f32 + buf * C::STAGE_F32;
    const int p = threadIdx.x;
    if (p < 2 * C::QUADS) {
      const bool is_q = p < C::QUADS;
      const int pp = is_q ? p : p - C::QUADS;
      const int rq = pp / (D / 8), c8 = (pp % (D / 8)) * 8;
      uint16_t* plain = base + (is_q ? 0 : C::PLAIN);
      uint16_t* trans = base + 2 * C::PLAIN + (is_q ? 0 : C::TRANS);
#pragma unroll
      for (int u = 0; u < 4; ++u) *reinterpret_cast<uint4*>(plain + (4 * rq + u) * C::ROW + c8) = st[u];
      const int pos = swap23(4 * rq);
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int wd = dd >> 1;
        const uint32_t a0 = word_of(st[0], wd), a1 = word_of(st[1], wd);
        const uint32_t a2 = word_of(st[2], wd), a3 = word_of(st[3], wd);
        uint2 out;
        if (dd & 1) {
          out.x = (a0 >> 16) | (a1 & 0xFFFF0000u);
          out.y = (a2 >> 16) | (a3 & 0xFFFF0000u);
        } else {
          out.x = (a0 & 0xFFFFu) | (a1 << 16);
          out.y = (a2 & 0xFFFFu) | (a3 << 16);
        }
        *reinterpret_cast<uint2*>(trans + (c8 + dd) * C::TROW + pos) = out;
      }
    }
    if (threadIdx.x < C::QT) {
      fb[threadIdx.x] = st_l;
      fb[C::QT + threadIdx.x] = st_d;
      reinterpret_cast<int*>(fb)[2 * C::QT + threadIdx.x] = st_r;
    }
  };

  if (n_qt > 0) {
    load_stage(mq_lo);
    store_stage(0);
  }
  __syncthreads();
  for (int it = 0; it < n_qt; ++it) {
    const int mt = mq_lo + it * C::QT;
    if (it + 1 < n_qt) load_stage(mt + C::QT);
    const uint16_t* Qs = lds_u16 + (it & 1) * C::STAGE_U16;
    const uint16_t* Os = Qs + C::PLAIN;
    const uint16_t* Qt = Qs + 2 * C::PLAIN;
    const uint16_t* Ot = Qt + C::TRANS;
    const float* fb = lds_f32 + (it & 1) * C::STAGE_F32;
    const int r_tlo = mt / g.grp, r_thi = (min(mt + C::QT, mq_hi) - 1) / g.grp;
    if (j0w <= r_thi && j0w < key_end) {
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const int off = col * C::ROW + ks * 16 + hl * 8;
        s = mfma32x32x16(as_bf16x8(*reinterpret_cast<const uint4*>(Qs + off)), kf[ks], s);
        dp = mfma32x32x16(as_bf16x8(*reinterpret_cast<const uint4*>(Os + off)), vf[ks], dp);
      }
      const bool need_mask = j0w + 31 > r_tlo;
      float p[16], ds[16];
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int row0 = i4 * 8 + hl * 4;
        const float4 l4 = *reinterpret_cast<const float4*>(fb + row0);
        const float4 d4 = *reinterpret_cast<const float4*>(fb + C::QT + row0);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
        int rv[4] = {0, 0, 0, 0};
        if (need_mask) {
          const int4 r4 = *reinterpret_cast<const int4*>(reinterpret_cast<const int*>(fb) + 2 * C::QT + row0);
          rv[0] = r4.x;
          rv[1] = r4.y;
          rv[2] = r4.z;
          rv[3] = r4.w;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = 4 * i4 + u;
          float pv = fast_exp2(s[i] * g.c2 - lv[u]);
          if (need_mask && my_key > rv[u]) pv = 0.0f;
          p[i] = pv;
          ds[i] = pv * (dp[i] - dv4[u]);
        }
      }
      bf16x8 pf[2], dsf[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        uint4 u, v;
        u.x = pack_bf16x2(p[8 * h2 + 0], p[8 * h2 + 1]);
        u.y = pack_bf16x2(p[8 * h2 + 2], p[8 * h2 + 3]);
        u.z = pack_bf16x2(p[8 * h2 + 4], p[8 * h2 + 5]);
        u.w = pack_bf16x2(p[8 * h2 + 6], p[8 * h2 + 7]);
        v.x = pack_bf16x2(ds[8 * h2 + 0], ds[8 * h2 + 1]);
        v.y = pack_bf16x2(ds[8 * h2 + 2], ds[8 * h2 + 3]);
        v.z = pack_bf16x2(ds[8 * h2 + 4], ds[8 * h2 + 5]);
        v.w = pack_bf16x2(ds[8 * h2 + 6], ds[8 * h2 + 7]);
        pf[h2] = as_bf16x8(u);
        dsf[h2] = as_bf16x8(v);
      }
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int off = (dt * 32 + col) * C::TROW + h2 * 16 + hl * 8;
          dv[dt] = mfma32x32x16(as_bf16x8(*reinterpret_cast<const uint4*>(Ot + off)), pf[h2], dv[dt]);
          dk[dt] = mfma32x32x16(as_bf16x8(*reinterpret_cast<const uint4*>(Qt + off)), dsf[h2], dk[dt]);
        }
      }
    }
    if (it + 1 < n_qt) store_stage((it + 1) & 1);
    __syncthreads();
  }

  if (my_key >= key_end) return;
  float* dkp = dk_r + kvrow * D;
  float* dvp = dv_r + kvrow * D;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = dt * 32 + i4 * 8 + hl * 4;
      float4 a = *reinterpret_cast<float4*>(dkp + d0);
      float4 b = *reinterpret_cast<float4*>(dvp + d0);
      a.x += dk[dt][4 * i4 + 0] * g.tau;
      a.y += dk[dt][4 * i4 + 1] * g.tau;
      a.z += dk[dt][4 * i4 + 2] * g.tau;
      a.w += dk[dt][4 * i4 + 3] * g.tau;
      b.x += dv[dt][4 * i4 + 0];
      b.y += dv[dt][4 * i4 + 1];
      b.z += dv[dt][4 * i4 + 2];
      b.w += dv[dt][4 * i4 + 3];
      *reinterpret_cast<float4*>(dkp + d0) = a;
      *reinterpret_cast<float4*>(dvp + d0) = b;
    }
}

hipError_t launch_dkdv_bf16(const Geom& g, const AttnPtrs& a, int key_hi, hipStream_t s) {
  if (key_hi <= 0) return hipSuccess;
  const int n_kt = (key_hi + KvCfg<128>::KEYS - 1) / KvCfg<128>::KEYS;
  const int64_t n = (int64_t)g.K * g.Hkv * n_kt;
  const dim3 grid((unsigned)xcd_grid(n)), block(256);
  const uint16_t *q = (const uint16_t*)a.q, *kr = (const uint16_t*)a.k_r, *vr = (const uint16_t*)a.v_r;
  const uint16_t* dO = (const uint16_t*)a.d_o;
  if (g.dqk == 64)
    hipLaunchKernelGGL(dkdv_bf16<64>, grid, block, 0, s, g, key_hi, q, kr, vr, dO, a.lse, a.Dvec, a.dk_r,
                       a.dv_r);
  else
    hipLaunchKernelGGL(dkdv_bf16<128>, grid, block, 0, s, g, key_hi, q, kr, vr, dO, a.lse, a.Dvec, a.dk_r,
                       a.dv_r);
  return hipGetLastError();
}

}  // namespace rr
