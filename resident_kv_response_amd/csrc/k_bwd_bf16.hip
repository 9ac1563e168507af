// bf16 response-only backward on MFMA (gfx950).
//
// Source of the contract: ai.thesatyajit.com/articles/longstraw-2m-rl, sections "The
// move: change the graph boundary" (the resident prompt state is a stop-gradient: only
// the direct response gradient is formed) and "Two incompatible architectures, same
// transaction" (response blocks replayed in reverse; K/V gradient storage only for
// what a response backward touches).  No kernel here reads or writes a prompt gradient.
//
// dq_partials_bf16: query-parallel, one workgroup per (k, g, part, 256-row tile) like
// the forward; per 32-key subtile S^T = K Q^T and dP^T = V dO^T - D (2 x D/16 MFMAs, the
// second accumulation starting from -D), p = 2^(S c2 - lse2), dS = p (dP - D) rounded to
// bf16, dQ^T += K^T dS^T (D/16 MFMAs).
// Writes one dQ partial per part; the partials are summed in part order afterwards.
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

#ifndef RR_DQ_WAVES
#define RR_DQ_WAVES 8
#endif

template <int D>
struct DqCfg {
  static constexpr int WAVES = RR_DQ_WAVES;
  static constexpr int BM = WAVES * 32;          // query rows per workgroup (32 per wave)
  static constexpr int BN = 128;                 // keys per LDS stage
  static constexpr int NSUB = BN / 32;
  static constexpr int KS = D / 16, DT = D / 32;
  static constexpr int TILE = BN * D * 2;
};

// One 32-key subtile of the dQ accumulation for this wave's 32 rows.
// The dP^T accumulation starts from dinit (every element -D of the lane's row), so the
// MFMAs deliver dP - D directly and dS = P (dP - D) is one multiply per element.
template <bool MASK, int D>
__device__ __forceinline__ void dq_subtile(const Frag<D>& fr, const char* Kt, const char* Vt, int sub,
                                           int rel, int lim,
                                           float c2, float lse2, const f32x16& dinit,
                                           const bf16x8 (&qf)[D / 16], const bf16x8 (&of)[D / 16],
                                           f32x16 (&acc)[D / 32]) {
  constexpr int KS = D / 16, DT = D / 32;
  const int hl = (threadIdx.x & 63) >> 5;
  f32x16 s, dp = dinit;
#pragma unroll
  for (int i = 0; i < 16; ++i) s[i] = 0.0f;
  prio_mfma();
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bf16x8 ak = fr.row(Kt, sub, ks);
    const bf16x8 av = fr.row(Vt, sub, ks);
    s = mfma32x32x16(ak, qf[ks], s);
    dp = mfma32x32x16(av, of[ks], dp);
  }
  prio_valu();
  float ds[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float p = fast_exp2(fmaf(s[i], c2, -lse2));
    if (MASK) {
      const int key = rel + (i >> 2) * 8 + hl * 4 + (i & 3);
      if (key > lim) p = 0.0f;
    }
    ds[i] = p * dp[i];
  }
  bf16x8 dsf[2];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    uint4 u;
    u.x = pack_bf16x2(ds[8 * h2 + 0], ds[8 * h2 + 1]);
    u.y = pack_bf16x2(ds[8 * h2 + 2], ds[8 * h2 + 3]);
    u.z = pack_bf16x2(ds[8 * h2 + 4], ds[8 * h2 + 5]);
    u.w = pack_bf16x2(ds[8 * h2 + 6], ds[8 * h2 + 7]);
    dsf[h2] = as_bf16x8(u);
  }
  prio_mfma();
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
      acc[dt] = mfma32x32x16(fr.trans_frag(Kt, sub, h2, dt), dsf[h2], acc[dt]);
  prio_valu();
}

template <int D>
__global__ __launch_bounds__(64 * RR_DQ_WAVES, 1) void dq_partials_bf16(
    Geom g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_p,
    const uint16_t* __restrict__ v_p, const uint16_t* __restrict__ k_r,
    const uint16_t* __restrict__ v_r, const uint16_t* __restrict__ d_o,
    const float* __restrict__ lse, const float* __restrict__ Dvec, float* __restrict__ dq_part) {
  using C = DqCfg<D>;
  constexpr int KS = C::KS, DT = C::DT;
  __shared__ __attribute__((aligned(1024))) char buf0[2 * C::TILE];   // K tile, V tile
  __shared__ __attribute__((aligned(1024))) char buf1[2 * C::TILE];

  const TileWork w = decode_tile_work(g, C::BM);
  if (!w.ok) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hl = lane >> 5, col = lane & 31;
  const int m_hi = g.row_hi * g.grp;
  const int r_first = w.m0 / g.grp;
  const int r_top = (min(m_hi, w.m0 + C::BM) - 1) / g.grp;
  const int rl = g.r_len[w.k];

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
  const int n_keys = (r_first >= rl || (resp && !g.resp_keys)) ? 0 : (int)(key1 - key0);
  const int n_stages = (n_keys + C::BN - 1) / C::BN;
  const int64_t sb = stride * 2;
  const uint16_t* kc = kb + key0 * stride;
  const uint16_t* vc = vb + key0 * stride;
  DirectLoad<D, C::BN, C::WAVES> dl;
  dl.init(sb);
  if (n_stages > 0) {
    dl.issue(buf0, kc, 0, n_keys, sb);
    dl.issue(buf0 + C::TILE, vc, 0, n_keys, sb);
  }
  Frag<D> fr;
  fr.init();

  const int m = w.m0 + wave * 32 + col;
  const int r = m / g.grp, h = w.g * g.grp + m % g.grp;
  const bool valid = m < m_hi && r < rl;
  const int lim = resp ? min(r, n_keys - 1) : n_keys - 1;
  const int64_t row = ((int64_t)w.k * g.R + r) * g.Hq + h;
  const int64_t orow = m < m_hi ? ((int64_t)w.part * g.K * g.R * g.Hq + row) : -1;
  const float lse2 = valid ? lse[row] * kLog2e : INFINITY;
  const float dvv = valid ? Dvec[row] : 0.0f;
  f32x16 dinit;
#pragma unroll
  for (int i = 0; i < 16; ++i) dinit[i] = -dvv;
  bf16x8 qf[KS], of[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = as_bf16x8(valid ? *reinterpret_cast<const uint4*>(q + row * D + ks * 16 + hl * 8)
                             : make_uint4(0, 0, 0, 0));
    of[ks] = as_bf16x8(valid ? *reinterpret_cast<const uint4*>(d_o + row * D + ks * 16 + hl * 8)
                             : make_uint4(0, 0, 0, 0));
  }
  int wmin = lim, wmax = lim;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    wmin = min(wmin, __shfl_xor(wmin, off, 64));
    wmax = max(wmax, __shfl_xor(wmax, off, 64));
  }

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.0f;

  auto stage = [&](const char* cur, char* nxt, int it) {
    wait_vmcnt0();
    __syncthreads();
    if (it + 1 < n_stages) {
      const int64_t nk0 = (int64_t)(it + 1) * C::BN;
      dl.issue(nxt, kc, nk0, n_keys, sb);
      dl.issue(nxt + C::TILE, vc, nk0, n_keys, sb);
    }
    const char* Kt = cur;
    const char* Vt = cur + C::TILE;
#pragma unroll
    for (int sub = 0; sub < C::NSUB; ++sub) {
      const int rel = it * C::BN + sub * 32;
      if (rel > wmax) break;
      if (rel + 31 > wmin)
        dq_subtile<true, D>(fr, Kt, Vt, sub, rel, lim, g.c2, lse2, dinit, qf, of, acc);
      else
        dq_subtile<false, D>(fr, Kt, Vt, sub, rel, lim, g.c2, lse2, dinit, qf, of, acc);
    }
  };
  for (int it = 0; it < n_stages; it += 2) {
    stage(buf0, buf1, it);
    if (it + 1 < n_stages) stage(buf1, buf0, it + 1);
  }

  if (orow < 0) return;
  const float sc = valid ? g.tau : 0.0f;
  float* dst = dq_part + orow * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = dt * 32 + i4 * 8 + hl * 4;
      *reinterpret_cast<float4*>(dst + d0) =
          make_float4(acc[dt][4 * i4 + 0] * sc, acc[dt][4 * i4 + 1] * sc, acc[dt][4 * i4 + 2] * sc,
                      acc[dt][4 * i4 + 3] * sc);
    }
}

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

hipError_t launch_dq_ring_bf16(const Geom& g, const AttnPtrs& a, hipStream_t s);

hipError_t launch_dq_partials_bf16(const Geom& g, const AttnPtrs& a, hipStream_t s) {
#ifndef RR_DQ_OLD
  return launch_dq_ring_bf16(g, a, s);
#endif
  const int64_t n = tile_work_count(g, DqCfg<128>::BM);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)xcd_grid(n)), block(64 * DqCfg<128>::WAVES);
  const uint16_t *q = (const uint16_t*)a.q, *kp = (const uint16_t*)a.k_p, *vp = (const uint16_t*)a.v_p;
  const uint16_t *kr = (const uint16_t*)a.k_r, *vr = (const uint16_t*)a.v_r, *dO = (const uint16_t*)a.d_o;
  if (g.dqk == 64)
    hipLaunchKernelGGL(dq_partials_bf16<64>, grid, block, 0, s, g, q, kp, vp, kr, vr, dO, a.lse, a.Dvec,
                       a.dq_part);
  else
    hipLaunchKernelGGL(dq_partials_bf16<128>, grid, block, 0, s, g, q, kp, vp, kr, vr, dO, a.lse, a.Dvec,
                       a.dq_part);
  return hipGetLastError();
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
