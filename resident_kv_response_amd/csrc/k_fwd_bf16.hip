// bf16 forward partials on MFMA (gfx950).
//
// One workgroup = one (response k, KV head g, part, 256-row tile).  A part is one prompt
// chunk [c*chunk, (c+1)*chunk) or the response's own causal keys; each part keeps its own
// softmax statistics (running max m, running sum l) and writes O_c = O~_c / l and
// lse_c = m + ln l, which are then composed exactly (ai.thesatyajit.com/articles/
// longstraw-2m-rl, section "Two incompatible architectures, same transaction").
//
// Rows: flattened m = r * grp + hh over the grp query heads that read KV head g, so one
// K/V tile feeds all of them.  8 waves x 32 rows (two waves per SIMD); each wave keeps
// its Q fragments and its O^T accumulators (d x rows, fp32) in registers for the whole
// part.
//
// K/V stream: 128-key stages loaded straight from global memory into LDS (no register
// staging), two buffers, the next stage's loads in flight while the current one is used.
// Per 32-key subtile and 32-row N-tile: S^T = K Q^T (D/16 MFMAs, K row fragments),
// base-2 online softmax with a lazy rescale (the reference maximum only moves when a
// row's maximum grows by more than 2^8, so every p <= 256), P^T rounded to bf16 straight
// from the C registers (the running sum l adds up those rounded values, so the
// normaliser is the sum of exactly the weights the PV product uses), O^T += V^T P^T
// (D/16 MFMAs, V^T fragments by transposing LDS reads).
//
// Stages whose keys are visible to every row of the wave run a software pipeline: the
// S^T MFMAs of subtile j+1 and the PV MFMAs of subtile j-1 are issued between short runs
// of the softmax of subtile j, so the matrix cores and the vector ALUs work at the same
// time.  Stages near the causal diagonal or a chunk end take the masked path.
#include "k_attn_tile.h"
#include "k_lds.h"
#include "kernels.h"

namespace rr {

constexpr float kRescaleThreshold = 8.0f;   // log2 of the largest p between rescales

#ifndef RR_FWD_WAVES
#define RR_FWD_WAVES 8
#endif
#ifndef RR_FWD_NT
#define RR_FWD_NT 1
#endif

template <int D>
struct FwdCfg {
  static constexpr int WAVES = RR_FWD_WAVES;
  static constexpr int NT = RR_FWD_NT;           // 32-row N-tiles per wave
  static constexpr int ROWS_W = 32 * NT;
  static constexpr int BM = WAVES * ROWS_W;      // query rows per workgroup
  static constexpr int BN = 128;                 // keys per LDS stage
  static constexpr int NSUB = BN / 32;
  static constexpr int KS = D / 16, DT = D / 32;
  static constexpr int TILE = BN * D * 2;        // bytes of one [BN][D] bf16 tile
};

template <int D, int NT>
__device__ __forceinline__ void scores_T(const Frag<D>& fr, const char* Kt, int sub,
                                         const bf16x8 (&qf)[NT][D / 16], f32x16 (&s)[NT]) {
  constexpr int KS = D / 16;
  bf16x8 kf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kf[ks] = fr.row(Kt, sub, ks);
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[t][i] = 0.0f;
  prio_mfma();
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int t = 0; t < NT; ++t) s[t] = mfma32x32x16(kf[ks], qf[t][ks], s[t]);
  prio_valu();
}

template <bool MASK, int D, int NT>
__device__ __forceinline__ void online_softmax(f32x16 (&s)[NT], const int (&lim)[NT], int rel,
                                               float c2, float (&m_run)[NT], float (&l_run)[NT],
                                               f32x16 (&acc)[NT][D / 32], bf16x8 (&pf)[NT][2]) {
  constexpr int DT = D / 32;
  const int hl = (threadIdx.x & 63) >> 5;
  float m_new[NT];
  bool grow = false;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (MASK) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = rel + (i >> 2) * 8 + hl * 4 + (i & 3);
        if (key > lim[t]) s[t][i] = -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(s[t][0], s[t][1]), s[t][2]);
#pragma unroll
    for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, s[t][i]), s[t][i + 1]);
    mx = fmaxf(mx, s[t][15]);
    mx = pair_max(mx);
    m_new[t] = fmaxf(m_run[t], mx * c2);
    grow |= m_new[t] > m_run[t] + kRescaleThreshold;
  }
  if (__any(grow)) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float alpha = fast_exp2(m_run[t] - m_new[t]);
      l_run[t] *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][dt][i] *= alpha;
      m_run[t] = m_new[t];
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = fast_exp2(fmaf(s[t][i], c2, -m_run[t]));
    float ls = 0.0f;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      uint4 u;
      u.x = pack_bf16x2(p[8 * h2 + 0], p[8 * h2 + 1]);
      u.y = pack_bf16x2(p[8 * h2 + 2], p[8 * h2 + 3]);
      u.z = pack_bf16x2(p[8 * h2 + 4], p[8 * h2 + 5]);
      u.w = pack_bf16x2(p[8 * h2 + 6], p[8 * h2 + 7]);
      pf[t][h2] = as_bf16x8(u);
      ls = sum_bf16x8(u, ls);
    }
    l_run[t] += ls;
  }
}

template <int D, int NT>
__device__ __forceinline__ void pv_accumulate(const Frag<D>& fr, const char* Vt, int sub,
                                              const bf16x8 (&pf)[NT][2], f32x16 (&acc)[NT][D / 32]) {
  constexpr int DT = D / 32;
  bf16x8 vf[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) vf[dt][h2] = fr.trans_frag(Vt, sub, h2, dt);
  prio_mfma();
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t][dt] = mfma32x32x16(vf[dt][h2], pf[t][h2], acc[t][dt]);
  prio_valu();
}

// Softmax of one unmasked 32-key subtile (one 32-row N-tile): P^T as bf16 MFMA operands
// in pf, and alpha, the factor the accumulators must be scaled by when the reference
// maximum moved (returned wave-uniform flag; alpha = 1 otherwise).  Branch-free, so it
// can share a basic block with the MFMAs it is scheduled against.
__device__ __forceinline__ bool softmax_plain(const f32x16& s, float c2, float& m_run, float& l_run,
                                              float& alpha, bf16x8 (&pf)[2]) {
  float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
  for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, s[i]), s[i + 1]);
  mx = fmaxf(mx, s[15]);
  mx = pair_max(mx);
  const float m_new = fmaxf(m_run, mx * c2);
  const bool grow = __any(m_new > m_run + kRescaleThreshold);
  const float m_use = grow ? m_new : m_run;
  alpha = fast_exp2(m_run - m_use);
  m_run = m_use;
  float p[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) p[i] = fast_exp2(fmaf(s[i], c2, -m_use));
  float ls = 0.0f;
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    uint4 u;
    u.x = pack_bf16x2(p[8 * h2 + 0], p[8 * h2 + 1]);
    u.y = pack_bf16x2(p[8 * h2 + 2], p[8 * h2 + 3]);
    u.z = pack_bf16x2(p[8 * h2 + 4], p[8 * h2 + 5]);
    u.w = pack_bf16x2(p[8 * h2 + 6], p[8 * h2 + 7]);
    pf[h2] = as_bf16x8(u);
    ls = sum_bf16x8(u, ls);
  }
  l_run = fmaf(l_run, alpha, ls);
  return grow;
}

template <int D>
__device__ __forceinline__ void scale_acc(f32x16 (&acc)[D / 32], float alpha) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;
}

// S^T of subtile `sub` for the wave's NT N-tiles: each K row fragment is read once and
// feeds NT MFMAs.
template <int D, int NT>
__device__ __forceinline__ void mma_scores(const Frag<D>& fr, const char* Kt, int sub,
                                           const bf16x8 (&qf)[NT][D / 16], f32x16 (&s)[NT]) {
  bf16x8 kf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) kf[ks] = fr.row(Kt, sub, ks);
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[t][i] = 0.0f;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
    for (int t = 0; t < NT; ++t) s[t] = mfma32x32x16(kf[ks], qf[t][ks], s[t]);
}

// O^T += V^T P^T of subtile `sub` for the wave's NT N-tiles (each V^T fragment feeds NT
// MFMAs).
template <int D, int NT>
__device__ __forceinline__ void mma_pv(const Frag<D>& fr, const char* Vt, int sub, const bf16x8 (&pf)[NT][2],
                                       f32x16 (&acc)[NT][D / 32]) {
  bf16x8 vf[D / 32][2];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) vf[dt][h2] = fr.trans_frag(Vt, sub, h2, dt);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t][dt] = mfma32x32x16(vf[dt][h2], pf[t][h2], acc[t][dt]);
}

// Softmax of the NT tiles of one subtile; true when any reference maximum moved (the
// accumulators of tile t must then be scaled by alpha[t], which is 1 for tiles that did
// not move).
template <int NT>
__device__ __forceinline__ bool softmax_tiles(const f32x16 (&s)[NT], float c2, float (&m_run)[NT],
                                              float (&l_run)[NT], float (&alpha)[NT], bf16x8 (&pf)[NT][2]) {
  bool grow = false;
#pragma unroll
  for (int t = 0; t < NT; ++t) grow |= softmax_plain(s[t], c2, m_run[t], l_run[t], alpha[t], pf[t]);
  return grow;
}

template <int D, int NT>
__device__ __forceinline__ void scale_tiles(f32x16 (&acc)[NT][D / 32], const float (&alpha)[NT]) {
#pragma unroll
  for (int t = 0; t < NT; ++t) scale_acc<D>(acc[t], alpha[t]);
}

// Schedules of the pipelined stage's basic blocks: (D/16) K-fragment reads and D/16 * NT
// MFMAs per S^T, (D/8) V^T reads and D/16 * NT MFMAs per PV.  Operand reads run a few
// MFMAs ahead of their use (not all up front, which would hold every fragment in
// registers at once), and each MFMA is followed by a share of the softmax's vector work.
template <int D, int NT>
__device__ __forceinline__ void sched_s_softmax() {      // S(j+1) with softmax(j)
  constexpr int NM = D / 16 * NT;
  RR_SCHED_GROUP(RR_SG_DS_READ, 4);
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    RR_SCHED_GROUP(RR_SG_MFMA, 1);
    if (i % NT == NT - 1 && i / NT < D / 16 - 4) RR_SCHED_GROUP(RR_SG_DS_READ, 1);
    RR_SCHED_GROUP(RR_SG_VALU, NT == 1 ? 9 : 7);
  }
}
template <int D, int NT>
__device__ __forceinline__ void sched_s_pv_softmax() {   // S(j+1) and PV(j-1) with softmax(j)
  constexpr int NM = D / 8 * NT, READS = D / 16 - 4 + D / 8, PER = NT == 1 ? 2 : 1;
  RR_SCHED_GROUP(RR_SG_DS_READ, 4);
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    RR_SCHED_GROUP(RR_SG_MFMA, 1);
    if (i < READS / PER) RR_SCHED_GROUP(RR_SG_DS_READ, PER);
    RR_SCHED_GROUP(RR_SG_VALU, NT == 1 ? 5 : 4);
  }
}
template <int D, int NT>
__device__ __forceinline__ void sched_pv_softmax() {     // PV(j-1) with softmax(j)
  constexpr int NM = D / 16 * NT, READS = D / 8 - 6, PER = NT == 1 ? 2 : 1;
  RR_SCHED_GROUP(RR_SG_DS_READ, 6);
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    RR_SCHED_GROUP(RR_SG_MFMA, 1);
    if (i < READS / PER) RR_SCHED_GROUP(RR_SG_DS_READ, PER);
    RR_SCHED_GROUP(RR_SG_VALU, NT == 1 ? 9 : 8);
  }
}

template <int D>
__global__ __launch_bounds__(64 * RR_FWD_WAVES, 1) void fwd_partials_bf16(
    Geom g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_p,
    const uint16_t* __restrict__ v_p, const uint16_t* __restrict__ k_r,
    const uint16_t* __restrict__ v_r, float* __restrict__ part_o, float* __restrict__ part_lse) {
  using C = FwdCfg<D>;
  constexpr int NT = C::NT, KS = C::KS, DT = C::DT;
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

  const int64_t sb = stride * 2;                  // bytes between consecutive keys
  const uint16_t* kc = kb + key0 * stride;          // part-relative streams
  const uint16_t* vc = vb + key0 * stride;
  DirectLoad<D, C::BN, C::WAVES> dl;
  dl.init(sb);
  Frag<D> fr;
  fr.init();
  if (n_stages > 0) {
    dl.issue(buf0, kc, 0, n_keys, sb);
    dl.issue(buf0 + C::TILE, vc, 0, n_keys, sb);
  }

  int lim[NT];
  bool valid[NT];
  int64_t orow[NT];
  bf16x8 qf[NT][KS];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int m = w.m0 + wave * C::ROWS_W + t * 32 + col;
    const int r = m / g.grp, h = w.g * g.grp + m % g.grp;
    valid[t] = m < m_hi && r < rl;
    lim[t] = resp ? min(r, n_keys - 1) : n_keys - 1;
    orow[t] = m < m_hi ? (((int64_t)w.part * g.K + w.k) * g.R + r) * g.Hq + h : -1;
    const uint16_t* qrow = q + (((int64_t)w.k * g.R + r) * g.Hq + h) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[t][ks] = as_bf16x8(valid[t] ? *reinterpret_cast<const uint4*>(qrow + ks * 16 + hl * 8)
                                     : make_uint4(0, 0, 0, 0));
  }
  int wmin = min(lim[0], lim[NT - 1]), wmax = max(lim[0], lim[NT - 1]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    wmin = min(wmin, __shfl_xor(wmin, off, 64));
    wmax = max(wmax, __shfl_xor(wmax, off, 64));
  }

  f32x16 acc[NT][DT];
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    m_run[t] = kNegBig;
    l_run[t] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[t][dt][i] = 0.0f;
  }

  // one stage: wait for its loads, prefetch the next stage into the other buffer, then
  // four 32-key subtiles with the next subtile's scores issued ahead of the softmax
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
    const int rel0 = it * C::BN;
    if (rel0 > wmax) return;
    if (C::NSUB == 4 && rel0 + C::BN - 1 <= wmin) {
      // every key of the stage is visible to every row of the wave: software-pipelined
      // subtiles, S(j+1) and PV(j-1) on the matrix cores while the softmax of j runs
      f32x16 sa[NT], sb[NT];
      bf16x8 pa[NT][2], pb[NT][2];
      float alpha[NT];
      mma_scores<D, NT>(fr, Kt, 0, qf, sa);
      mma_scores<D, NT>(fr, Kt, 1, qf, sb);
      bool grow = softmax_tiles<NT>(sa, g.c2, m_run, l_run, alpha, pa);
      sched_s_softmax<D, NT>();
      if (grow) scale_tiles<D, NT>(acc, alpha);
      mma_scores<D, NT>(fr, Kt, 2, qf, sa);
      mma_pv<D, NT>(fr, Vt, 0, pa, acc);
      grow = softmax_tiles<NT>(sb, g.c2, m_run, l_run, alpha, pb);
      sched_s_pv_softmax<D, NT>();
      if (grow) scale_tiles<D, NT>(acc, alpha);
      mma_scores<D, NT>(fr, Kt, 3, qf, sb);
      mma_pv<D, NT>(fr, Vt, 1, pb, acc);
      grow = softmax_tiles<NT>(sa, g.c2, m_run, l_run, alpha, pa);
      sched_s_pv_softmax<D, NT>();
      if (grow) scale_tiles<D, NT>(acc, alpha);
      mma_pv<D, NT>(fr, Vt, 2, pa, acc);
      grow = softmax_tiles<NT>(sb, g.c2, m_run, l_run, alpha, pb);
      sched_pv_softmax<D, NT>();
      if (grow) scale_tiles<D, NT>(acc, alpha);
      mma_pv<D, NT>(fr, Vt, 3, pb, acc);
      return;
    }
    f32x16 s_cur[NT];
    scores_T<D, NT>(fr, Kt, 0, qf, s_cur);
#pragma unroll
    for (int sub = 0; sub < C::NSUB; ++sub) {
      const int rel = rel0 + sub * 32;
      const bool has_next = sub + 1 < C::NSUB && rel + 32 <= wmax;
      f32x16 s_next[NT];
      if (has_next) scores_T<D, NT>(fr, Kt, sub + 1, qf, s_next);
      bf16x8 pf[NT][2];
      if (rel + 31 > wmin)
        online_softmax<true, D, NT>(s_cur, lim, rel, g.c2, m_run, l_run, acc, pf);
      else
        online_softmax<false, D, NT>(s_cur, lim, rel, g.c2, m_run, l_run, acc, pf);
      pv_accumulate<D, NT>(fr, Vt, sub, pf, acc);
      if (!has_next) break;
#pragma unroll
      for (int t = 0; t < NT; ++t) s_cur[t] = s_next[t];
    }
  };

  for (int it = 0; it < n_stages; it += 2) {
    stage(buf0, buf1, it);
    if (it + 1 < n_stages) stage(buf1, buf0, it + 1);
  }

#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float l = pair_sum(l_run[t]);
    if (orow[t] < 0) continue;
    const bool live = valid[t] && l > 0.0f;
    const float inv = live ? 1.0f / l : 0.0f;
    float* dst = part_o + orow[t] * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
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

hipError_t launch_fwd_ring_bf16(const Geom& g, const AttnPtrs& a, hipStream_t s);

hipError_t launch_fwd_partials_bf16(const Geom& g, const AttnPtrs& a, hipStream_t s) {
#ifndef RR_FWD_OLD
  return launch_fwd_ring_bf16(g, a, s);
#endif
  const int64_t n = tile_work_count(g, FwdCfg<128>::BM);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)xcd_grid(n)), block(64 * FwdCfg<128>::WAVES);
  const uint16_t *q = (const uint16_t*)a.q, *kp = (const uint16_t*)a.k_p, *vp = (const uint16_t*)a.v_p;
  const uint16_t *kr = (const uint16_t*)a.k_r, *vr = (const uint16_t*)a.v_r;
  if (g.dqk == 64)
    hipLaunchKernelGGL(fwd_partials_bf16<64>, grid, block, 0, s, g, q, kp, vp, kr, vr, a.part_o, a.part_lse);
  else
    hipLaunchKernelGGL(fwd_partials_bf16<128>, grid, block, 0, s, g, q, kp, vp, kr, vr, a.part_o, a.part_lse);
  return hipGetLastError();
}

}  // namespace rr
