// bf16 forward partials on MFMA (gfx950), continuous software pipeline over a ring of
// K/V stages.
//
// One workgroup = one (response k, KV head g, part, 256-row tile).  A part is one prompt
// chunk [c*chunk, (c+1)*chunk) or the response's own causal keys; each part keeps its own
// softmax statistics (running max m, running sum l) and writes O_c = O~_c / l and
// lse_c = m + ln l, which are then composed exactly (ai.thesatyajit.com/articles/
// longstraw-2m-rl, section "Two incompatible architectures, same transaction").
//
// Rows: flattened m = r * grp + hh over the grp query heads that read KV head g, so one
// K/V tile feeds all of them.  A wave owns NT 32-row tiles: 8 waves x 32 rows (two waves
// per SIMD, NT = 1) or 4 waves x 64 rows (one wave per SIMD, NT = 2, where every K or V
// fragment read from LDS feeds two MFMAs).  Each wave keeps its Q fragments and its O^T
// accumulators (d x rows, fp32) in registers for the whole part.
//
// K/V stream: 64-key stages in a ring of four LDS buffers, loaded straight from global
// memory into LDS two stages ahead; one barrier per stage.  The K and V tiles of the
// four stages are separate arrays and every read names its buffer at compile time, so the
// compiler can tell a read of one buffer from the direct loads still landing in another.
//
// Pipeline over 32-key subtiles u, per wave: block B(u) issues O^T += V^T P^T of subtile
// u-1 and S^T = K Q^T of subtile u+1 on the matrix cores (MFMAs with no dependence on the
// block's vector work) while the vector ALUs run the online softmax of subtile u (base 2,
// lazy rescale: the reference maximum only moves when a row's maximum grows by more than
// 2^8, so every p <= 256; P^T rounded to bf16 straight from the C registers, and the
// running sum l adds up exactly those rounded values).  The block is laid out by hand in
// slots (one fragment read two slots ahead, its MFMAs, a fixed share of the softmax),
// separated by scheduling barriers.  A rescale of the accumulators is applied at the end
// of the block, between PV(u-1) and PV(u).  The block sequence runs across stage
// boundaries, so every block carries the same balanced load.  Subtiles whose keys are
// visible to every row of the workgroup run this pipeline; the few near the causal
// diagonal or a chunk end run a masked, unpipelined path afterwards.
#include <type_traits>

#include "k_attn_tile.h"
#include "k_lds.h"
#include "k_ring.h"
#include "kernels.h"

namespace rr {

#ifndef RR_AHEAD
#define RR_AHEAD 2   // slots between a fragment's LDS read and its MFMA
#endif

namespace {

constexpr float kRingRescaleLog2 = 8.0f;   // masked path: log2 of the largest p between rescales
// Pipelined path: largest partial row sum (16 bf16 p values of one lane) accepted against
// the current reference maximum; it bounds every p the PV product consumes.
constexpr float kRingSumLimit = 4096.0f;

template <int D, int NT>
struct RingCfg {
  static constexpr int WAVES = 8 / NT;
  static constexpr int BM = WAVES * 32 * NT;            // query rows per workgroup
  static constexpr int BN = 64;                         // keys per stage
  static constexpr int KS = D / 16, DT = D / 32;
  static constexpr int TILE = BN * D * 2;               // bytes of one [BN][D] bf16 tile
  static constexpr int LOADS = 2 * (BN * D / 8) / (64 * WAVES);   // direct loads per wave per stage
};

template <int D, int NT>
__device__ __forceinline__ void ring_scores(const Frag<D>& fr, const char* Kt, int sub,
                                            const bf16x8 (&qf)[NT][D / 16], f32x16 (&s)[NT]) {
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) s[t][i] = 0.0f;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const bf16x8 kf = fr.row(Kt, sub, ks);
#pragma unroll
    for (int t = 0; t < NT; ++t) s[t] = mfma32x32x16(kf, qf[t][ks], s[t]);
  }
}

template <int D, int NT>
__device__ __forceinline__ void ring_pv(const FarFrags<D>& vo, const char* Vt, int sub,
                                        const bf16x8 (&pf)[NT][2], f32x16 (&acc)[NT][D / 32]) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const bf16x8 vf = vo.trans_frag(Vt, sub, h2, dt);
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t][dt] = mfma32x32x16(vf, pf[t][h2], acc[t][dt]);
    }
}

// Online softmax of one 32-key subtile of one tile (lane = query row, 16 of the subtile's
// keys per lane), unpipelined form for the masked path.  Returns the wave-uniform
// "reference maximum moved" flag; alpha is the factor the accumulators must then be
// scaled by (1 on rows whose maximum did not move).
__device__ __forceinline__ bool ring_softmax(const f32x16& s, float c2, float& m_run, float& l_run,
                                             float& alpha, bf16x8 (&pf)[2]) {
  float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
  for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, s[i]), s[i + 1]);
  mx = fmaxf(mx, s[15]);
  mx = pair_max(mx);
  const float m_new = fmaxf(m_run, mx * c2);
  const bool grow = __any(m_new > m_run + kRingRescaleLog2);
  const float m_use = grow ? m_new : m_run;
  alpha = fast_exp2(m_run - m_use);
  m_run = m_use;
  float ls = 0.0f;
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = fast_exp2(fmaf(s[8 * h2 + i], c2, -m_use));
    uint4 u;
    u.x = pack_bf16x2(p[0], p[1]);
    u.y = pack_bf16x2(p[2], p[3]);
    u.z = pack_bf16x2(p[4], p[5]);
    u.w = pack_bf16x2(p[6], p[7]);
    pf[h2] = as_bf16x8(u);
    ls = sum_bf16x8(u, ls);
  }
  l_run = fmaf(l_run, alpha, ls);
  return grow;
}

template <int D>
__device__ __forceinline__ void ring_scale(f32x16 (&acc)[D / 32], float alpha) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;
}

// One pipelined block, laid out by hand as NSLOT slots separated by scheduling
// barriers.  Slot i issues the LDS reads of slot i+RR_AHEAD's fragment, then the NT MFMAs
// of its own fragment, then a fixed share of the softmax of subtile u for every tile: the
// exponentials p = 2^(S c2 - m) against the current reference maximum m, one per slot (a
// pair in every other slot measured 0.7 % slower), each pair packed to bf16 and added to
// the lane's partial row sum ls at the slot of its second element.  With PV, even
// slots hold the K fragments of subtile u+1's scores and odd slots the V^T fragments of
// subtile u-1's PV.  The caller accepts the subtile when every lane's ls is at most
// kRingSumLimit (then every p is at most that, since all p >= 0); otherwise it redoes the
// subtile against the true running maximum (ring_redo).
template <int D, int NT, bool HAS_PV>
__device__ __forceinline__ void ring_block_body(const Frag<D>& fr, const FarFrags<D>& vo, const char* Kt,
                                                int subk, const char* Vt, int subv,
                                                const bf16x8 (&qf)[NT][D / 16], const f32x16 (&s)[NT],
                                                const bf16x8 (&pp)[NT][2], f32x16 (&acc)[NT][D / 32],
                                                float c2, const float (&m_run)[NT], float (&ls)[NT],
                                                f32x16 (&sn)[NT], bf16x8 (&pn)[NT][2]) {
  constexpr int KS = D / 16;
  constexpr int NSLOT = (HAS_PV ? 2 : 1) * KS;
  auto load = [&](int i) -> bf16x8 {
    if (HAS_PV && (i & 1)) {
      const int j = i >> 1;
      return vo.trans_frag(Vt, subv, j & 1, j >> 1);
    }
    return fr.row(Kt, subk, HAS_PV ? (i >> 1) : i);
  };
  bf16x8 frag[NSLOT];
#pragma unroll
  for (int i = 0; i < RR_AHEAD && i < NSLOT; ++i) frag[i] = load(i);
  uint32_t w[NT][8];
  float pe[NT][16];
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int t = 0; t < NT; ++t) ls[t] = 0.0f;
#pragma unroll
  for (int i = 0; i < NSLOT; ++i) {
    if (i + RR_AHEAD < NSLOT) frag[i + RR_AHEAD] = load(i + RR_AHEAD);
    if (HAS_PV && (i & 1)) {
      const int j = i >> 1;
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t][j >> 1] = mfma32x32x16(frag[i], pp[t][j & 1], acc[t][j >> 1]);
    } else {
      const int ks = HAS_PV ? (i >> 1) : i;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (ks == 0) {
#pragma unroll
          for (int e = 0; e < 16; ++e) sn[t][e] = 0.0f;
        }
        sn[t] = mfma32x32x16(frag[i], qf[t][ks], sn[t]);
      }
    }
    // this slot's share of the softmax, for every tile: one exponential per slot (in
    // order), and each pair packed and summed at the slot of its second element
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if (i == (e * NSLOT) / 16) {
          pe[t][e] = fast_exp2(fmaf(s[t][e], c2, -m_run[t]));
          asm volatile("" ::"v"(pe[t][e]));
        }
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (i == ((2 * k + 1) * NSLOT) / 16) {
          w[t][k] = pack_bf16x2(pe[t][2 * k], pe[t][2 * k + 1]);
          ls[t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[t][k]), one, ls[t], false);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    pn[t][0] = as_bf16x8(make_uint4(w[t][0], w[t][1], w[t][2], w[t][3]));
    pn[t][1] = as_bf16x8(make_uint4(w[t][4], w[t][5], w[t][6], w[t][7]));
  }
}

// Slow path of a pipelined subtile whose partial row sum exceeded the limit (and the
// first subtile of a part): move the reference to the true running maximum, and
// recompute P and the subtile's sum against it.  Returns alpha, the factor the running
// sum and the accumulators (which already hold PV of subtile u-1) must be scaled by.
__device__ __forceinline__ float ring_redo(const f32x16& s, float c2, float& m_run, float& ls,
                                           bf16x8 (&pn)[2]) {
  float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
  for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, s[i]), s[i + 1]);
  mx = fmaxf(mx, s[15]);
  mx = pair_max(mx);
  const float m_new = fmaxf(m_run, mx * c2);
  const float alpha = fast_exp2(m_run - m_new);
  ls = 0.0f;
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = fast_exp2(fmaf(s[8 * h2 + i], c2, -m_new));
    uint4 u;
    u.x = pack_bf16x2(p[0], p[1]);
    u.y = pack_bf16x2(p[2], p[3]);
    u.z = pack_bf16x2(p[4], p[5]);
    u.w = pack_bf16x2(p[6], p[7]);
    pn[h2] = as_bf16x8(u);
    ls = sum_bf16x8(u, ls);
  }
  m_run = m_new;
  return alpha;
}

}  // namespace

template <int D, int NT>
__global__ __launch_bounds__(512 / NT, 1) void fwd_partials_bf16(
    Geom g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_p,
    const uint16_t* __restrict__ v_p, const uint16_t* __restrict__ k_r,
    const uint16_t* __restrict__ v_r, float* __restrict__ part_o, float* __restrict__ part_lse) {
  using C = RingCfg<D, NT>;
  constexpr int KS = C::KS, DT = C::DT;
  // K tiles of the four stages first, then the V tiles: the K tiles then sit within the
  // 16-bit immediate offset of one base address, the V tiles within that of another.
  __shared__ __attribute__((aligned(1024))) char kt0[C::TILE];
  __shared__ __attribute__((aligned(1024))) char kt1[C::TILE];
  __shared__ __attribute__((aligned(1024))) char kt2[C::TILE];
  __shared__ __attribute__((aligned(1024))) char kt3[C::TILE];
  __shared__ __attribute__((aligned(1024))) char vt0[C::TILE];
  __shared__ __attribute__((aligned(1024))) char vt1[C::TILE];
  __shared__ __attribute__((aligned(1024))) char vt2[C::TILE];
  __shared__ __attribute__((aligned(1024))) char vt3[C::TILE];
  char* const KT[4] = {kt0, kt1, kt2, kt3};
  char* const VT[4] = {vt0, vt1, vt2, vt3};

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
  // Workgroup-uniform subtile counts: [0, n_full) is visible to every row of the
  // workgroup (its first row sees the fewest response keys), [n_full, n_sub) is masked.
  const int lim_min = resp ? min(r_first, n_keys - 1) : n_keys - 1;
  const int n_full = n_keys > 0 ? (lim_min + 1) / 32 : 0;
  const int n_sub = (n_keys + 31) / 32;
  const int n_stages = (n_keys + C::BN - 1) / C::BN;

  const int64_t sbytes = stride * 2;
  const uint16_t* kc = kb + key0 * stride;
  const uint16_t* vc = vb + key0 * stride;
  DirectLoadRows<D, C::BN, C::WAVES> dl;
  dl.init();
  Frag<D> fr;
  fr.init();
  FarFrags<D> vo;
  vo.template init<false, true>(fr);

  auto issue_stage = [&](int b, int s) {
    const int64_t off = (int64_t)s * C::BN * sbytes;
    const int rows = n_keys - s * C::BN;
    dl.issue(lds_addr(KT[b]), reinterpret_cast<const char*>(kc) + off, rows, (uint32_t)sbytes);
    dl.issue(lds_addr(VT[b]), reinterpret_cast<const char*>(vc) + off, rows, (uint32_t)sbytes);
  };
  auto issue_any = [&](int s) {
    switch (s & 3) {
      case 0: issue_stage(0, s); break;
      case 1: issue_stage(1, s); break;
      case 2: issue_stage(2, s); break;
      default: issue_stage(3, s); break;
    }
  };
  // Entering stage s: its loads are done (only stage s+1's may still be in flight), every
  // wave is past its reads of stage s-2's buffer, and stage s+2 is loaded into it.
  int entered = -1;
  auto enter_stage = [&](int s) {
    if (s + 1 < n_stages) wait_vmcnt_n<C::LOADS>(); else wait_vmcnt0();
    __syncthreads();
    if (s + 2 < n_stages) issue_any(s + 2);
    entered = s;
  };
  if (n_stages > 0) issue_any(0);
  if (n_stages > 1) issue_any(1);

  int lim[NT];
  bool valid[NT];
  int64_t orow[NT];
  bf16x8 qf[NT][KS];
  int wmax = -1;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int m = w.m0 + (wave * NT + t) * 32 + col;
    const int r = m / g.grp, h = w.g * g.grp + m % g.grp;
    valid[t] = m < m_hi && r < rl;
    lim[t] = resp ? min(r, n_keys - 1) : n_keys - 1;
    orow[t] = m < m_hi ? (int64_t)w.part * g.part_step + (((int64_t)w.k * g.R + r) * g.Hq + h) * g.row_step : -1;
    const uint16_t* qrow = q + (((int64_t)w.k * g.R + r) * g.Hq + h) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[t][ks] = as_bf16x8(valid[t] ? *reinterpret_cast<const uint4*>(qrow + ks * 16 + hl * 8)
                                     : make_uint4(0, 0, 0, 0));
    wmax = max(wmax, lim[t]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) wmax = max(wmax, __shfl_xor(wmax, off, 64));

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
  const float c2 = g.c2;

  if (n_keys > 0) enter_stage(0);

  if (n_full > 0) {
    f32x16 s[NT];
    ring_scores<D, NT>(fr, KT[0], 0, qf, s);    // S(0)
    bf16x8 pp[NT][2];                           // P(u-1)

    // Block B(u), u = J mod 8: PV(u-1) and S(u+1) on the matrix cores, softmax of u on the
    // vector ALUs; compile-time buffers.  The last block also computes S(n_full), which is
    // never used (the masked path recomputes it) and reads a buffer with no loads in flight.
    auto block = [&](auto jc, auto pvc, int u) {
      constexpr int J = decltype(jc)::value;
      constexpr bool HAS_PV = decltype(pvc)::value;
      constexpr int SX = ((J + 7) >> 1) & 3, SUBX = (J + 7) & 1;   // subtile u-1
      constexpr int SY = ((J + 1) >> 1) & 3, SUBY = (J + 1) & 1;   // subtile u+1
      constexpr int SN = (SY + 2) & 3;                              // stage u/2 + 3's buffer
      if (J & 1) {   // subtile u+1 starts stage (u+1)/2
        const int st = (u + 1) >> 1;
        if (st + 1 < n_stages) wait_vmcnt_n<C::LOADS>(); else wait_vmcnt0();
        __syncthreads();
        if (st + 2 < n_stages) issue_stage(SN, st + 2);
        entered = st;
      }
      bf16x8 pn[NT][2];
      float ls[NT];
      f32x16 sn[NT];
      ring_block_body<D, NT, HAS_PV>(fr, vo, KT[SY], SUBY, VT[SX], SUBX, qf, s, pp, acc, c2, m_run, ls, sn,
                                     pn);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        // the block's softmax results must be formed here, not sunk past the check below
        pin_operands(pn[t], ls[t]);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bool redo = __any(!(ls[t] <= kRingSumLimit));
        float alpha = 1.0f;
        if (redo) alpha = ring_redo(s[t], c2, m_run[t], ls[t], pn[t]);
        if (redo) ring_scale<D>(acc[t], alpha);
        l_run[t] = fmaf(l_run[t], alpha, ls[t]);
        pp[t][0] = pn[t][0];
        pp[t][1] = pn[t][1];
        s[t] = sn[t];
      }
    };
    using T = std::true_type;
    using F = std::false_type;
    block(std::integral_constant<int, 0>{}, F{}, 0);
    int u = 1;
    // straight-line groups of eight blocks (u = 8i+1 .. 8i+8), so that every block's
    // buffers are compile-time and one block's softmax feeds the next block directly
    for (; u + 8 <= n_full; u += 8) {
      block(std::integral_constant<int, 1>{}, T{}, u);
      block(std::integral_constant<int, 2>{}, T{}, u + 1);
      block(std::integral_constant<int, 3>{}, T{}, u + 2);
      block(std::integral_constant<int, 4>{}, T{}, u + 3);
      block(std::integral_constant<int, 5>{}, T{}, u + 4);
      block(std::integral_constant<int, 6>{}, T{}, u + 5);
      block(std::integral_constant<int, 7>{}, T{}, u + 6);
      block(std::integral_constant<int, 0>{}, T{}, u + 7);
    }
    if (u < n_full) block(std::integral_constant<int, 1>{}, T{}, u++);
    if (u < n_full) block(std::integral_constant<int, 2>{}, T{}, u++);
    if (u < n_full) block(std::integral_constant<int, 3>{}, T{}, u++);
    if (u < n_full) block(std::integral_constant<int, 4>{}, T{}, u++);
    if (u < n_full) block(std::integral_constant<int, 5>{}, T{}, u++);
    if (u < n_full) block(std::integral_constant<int, 6>{}, T{}, u++);
    if (u < n_full) block(std::integral_constant<int, 7>{}, T{}, u++);
    // PV of the last pipelined subtile
    const int ul = n_full - 1;
    switch ((ul >> 1) & 3) {
      case 0: ring_pv<D, NT>(vo, VT[0], ul & 1, pp, acc); break;
      case 1: ring_pv<D, NT>(vo, VT[1], ul & 1, pp, acc); break;
      case 2: ring_pv<D, NT>(vo, VT[2], ul & 1, pp, acc); break;
      default: ring_pv<D, NT>(vo, VT[3], ul & 1, pp, acc); break;
    }
  }

  // Masked subtiles near the causal diagonal or a chunk end (keys past a row's limit
  // are invisible to it).
  for (int u = n_full; u < n_sub; ++u) {
    const int st = u >> 1;
    while (entered < st) enter_stage(entered + 1);
    const int rel = u * 32;
    if (rel > wmax) continue;
    const int b = st & 3;
    const char* const kt = b == 0 ? kt0 : b == 1 ? kt1 : b == 2 ? kt2 : kt3;
    const char* const vt = b == 0 ? vt0 : b == 1 ? vt1 : b == 2 ? vt2 : vt3;
    f32x16 s[NT];
    ring_scores<D, NT>(fr, kt, u & 1, qf, s);
    bf16x8 pf[NT][2];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = rel + (i >> 2) * 8 + hl * 4 + (i & 3);
        if (key > lim[t]) s[t][i] = -INFINITY;
      }
      float alpha;
      if (ring_softmax(s[t], c2, m_run[t], l_run[t], alpha, pf[t])) ring_scale<D>(acc[t], alpha);
    }
    ring_pv<D, NT>(vo, vt, u & 1, pf, acc);
  }
  // The direct loads are not tracked by the compiler: none may still be writing LDS when
  // the workgroup ends (every issued stage has been entered and waited for by now; this
  // makes it unconditional).
  wait_vmcnt0();

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

// Launched with one 32-row tile per wave, two waves per SIMD.  Two tiles per wave (64
// rows, one wave per SIMD) halve LDS reads per MFMA; with the accumulators held in AGPRs
// that form is correct but 12 % slower on MI355X: the second wave of a SIMD hides more
// latency than the halved LDS traffic saves.
hipError_t launch_fwd_partials_bf16(const Geom& g, const AttnPtrs& a, hipStream_t s) {
  const uint16_t *q = (const uint16_t*)a.q, *kp = (const uint16_t*)a.k_p, *vp = (const uint16_t*)a.v_p;
  const uint16_t *kr = (const uint16_t*)a.k_r, *vr = (const uint16_t*)a.v_r;
  if (g.dqk == 64) {
    using C = RingCfg<64, 1>;
    const int64_t n = tile_work_count(g, C::BM);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL((fwd_partials_bf16<64, 1>), dim3((unsigned)xcd_grid(n)), dim3(64 * C::WAVES), 0, s, g, q,
                       kp, vp, kr, vr, a.part_o, a.part_lse);
  } else {
    using C = RingCfg<128, 1>;
    const int64_t n = tile_work_count(g, C::BM);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL((fwd_partials_bf16<128, 1>), dim3((unsigned)xcd_grid(n)), dim3(64 * C::WAVES), 0, s, g, q,
                       kp, vp, kr, vr, a.part_o, a.part_lse);
  }
  return hipGetLastError();
}

}  // namespace rr
