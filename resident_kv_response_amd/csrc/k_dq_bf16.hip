// bf16 dQ partials over the resident prompt chunks and the response's causal keys, on
// MFMA (gfx950), with a continuous software pipeline over a ring of K/V stages.
//
// Source of the contract: ai.thesatyajit.com/articles/longstraw-2m-rl, sections "The
// move: change the graph boundary" (the resident prompt state is a stop-gradient: only
// the direct response gradient is formed) and "Two incompatible architectures, same
// transaction" (the resident K/V pages get no gradient storage).  This kernel reads the
// prompt K/V and writes only dQ.
//
// Query-parallel like the forward: one workgroup per (response k, KV head g, part,
// 256-row tile), 8 waves x 32 flattened rows (m = r * grp + hh).  Per 32-key subtile u:
// S^T = K Q^T and dP^T = V dO^T - D (the second accumulation starts from -D), then
// p = 2^(S c2 - lse2) with the global lse, dS = p (dP - D) rounded to bf16, and
// dQ^T += K^T dS^T.  One dQ partial per part; the partials are summed in part order
// afterwards.
//
// K/V stream: 64-key stages in a ring of four LDS buffers (K tiles and V tiles as
// separate arrays), loaded straight from global memory two stages ahead; one barrier per
// stage.  Pipeline: block B(u) issues dQ^T += K^T dS^T of subtile u-1, then the S and dP
// MFMAs of subtile u+1 (which reuse the registers of S(u), dP(u)), while the vector ALUs
// turn S(u), dP(u) into dS(u): exponentials during the dQ MFMAs, products and packing
// during the S MFMAs.  The block is laid out by
// hand in slots (the LDS reads of a fragment two slots ahead of its MFMA), separated by
// scheduling barriers, and the block sequence runs across stage boundaries.  Subtiles
// visible to every row of the workgroup run this pipeline; those near the causal
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

template <int D>
struct DqRingCfg {
  static constexpr int WAVES = 8;
  static constexpr int BM = WAVES * 32;                 // query rows per workgroup
  static constexpr int BN = 64;                         // keys per stage
  static constexpr int KS = D / 16, DT = D / 32;
  static constexpr int TILE = BN * D * 2;               // bytes of one [BN][D] bf16 tile
  static constexpr int LOADS = 2 * (BN * D / 8) / (64 * WAVES);   // direct loads per wave per stage
};

// S^T and dP^T - D of one subtile (unpipelined form).
template <int D>
__device__ __forceinline__ void dqr_scores(const Frag<D>& fr, const FarFrags<D>& far, const char* Kt,
                                           const char* Vt, int sub, const bf16x8 (&qf)[D / 16],
                                           const bf16x8 (&of)[D / 16], const f32x16& dinit, f32x16& s,
                                           f32x16& dp) {
#pragma unroll
  for (int i = 0; i < 16; ++i) s[i] = 0.0f;
  dp = dinit;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    s = mfma32x32x16(fr.row(Kt, sub, ks), qf[ks], s);
    dp = mfma32x32x16(far.row_folded(Vt, sub, ks), of[ks], dp);
  }
}

// dQ^T += K^T dS^T of one subtile (unpipelined form).
template <int D>
__device__ __forceinline__ void dqr_dq(const Frag<D>& fr, const char* Kt, int sub, const bf16x8 (&dsf)[2],
                                       f32x16 (&acc)[D / 32]) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) acc[dt] = mfma32x32x16(fr.trans_frag(Kt, sub, h2, dt), dsf[h2], acc[dt]);
}

// One pipelined block, laid out by hand in slots separated by scheduling barriers.
// With PREV the slots are: D/16 dQ MFMAs of subtile u-1 (K^T fragments), carrying the
// exponentials p = 2^(S c2 - lse2) of subtile u (each p replaces its S value); D/16 S
// MFMAs of subtile u+1, carrying dS = p (dP - D) and the bf16 packing (dP(u) is still
// live there); D/16 dP MFMAs of subtile u+1.  Every slot first issues the LDS reads of
// the fragment two slots ahead.
template <int D, bool PREV>
__device__ __forceinline__ void dqr_block_body(const Frag<D>& fr, const FarFrags<D>& far, const char* Kx,
                                               int subx, const char* Ky, const char* Vy, int suby,
                                               const bf16x8 (&qf)[D / 16], const bf16x8 (&of)[D / 16],
                                               const f32x16& dinit, float c2, float lse2,
                                               const bf16x8 (&dsp)[2], f32x16 (&acc)[D / 32], f32x16& s,
                                               f32x16& dp, bf16x8 (&dsn)[2]) {
  constexpr int KS = D / 16;
  constexpr int NX = PREV ? KS : 0;          // dQ slots
  constexpr int NSLOT = NX + 2 * KS;
  auto load = [&](int i) -> bf16x8 {
    if (i < NX) return fr.trans_frag(Kx, subx, i & 1, i >> 1);
    const int j = i - NX;
    return j < KS ? fr.row(Ky, suby, j) : far.row_folded(Vy, suby, j - KS);
  };
  float p[16];
  uint32_t w[8];
  if (!PREV) {
    // first block: no dQ MFMAs to overlap, so the exponentials run up front
#pragma unroll
    for (int e = 0; e < 16; ++e) p[e] = fast_exp2(fmaf(s[e], c2, -lse2));
    __builtin_amdgcn_sched_barrier(0);
  }
  bf16x8 frag[NSLOT];
#pragma unroll
  for (int i = 0; i < RR_AHEAD && i < NSLOT; ++i) frag[i] = load(i);
#pragma unroll
  for (int i = 0; i < NSLOT; ++i) {
    if (i + RR_AHEAD < NSLOT) frag[i + RR_AHEAD] = load(i + RR_AHEAD);
    if (i < NX) {
      acc[i >> 1] = mfma32x32x16(frag[i], dsp[i & 1], acc[i >> 1]);
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if ((e * NX) / 16 == i) {
          p[e] = fast_exp2(fmaf(s[e], c2, -lse2));
          asm volatile("" ::"v"(p[e]));   // keeps the exponential in this slot
        }
    } else if (i < NX + KS) {
      const int ks = i - NX;
      if (ks == 0) {
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = 0.0f;
      }
      s = mfma32x32x16(frag[i], qf[ks], s);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if ((k * KS) / 8 == ks) {
          w[k] = pack_bf16x2(p[2 * k] * dp[2 * k], p[2 * k + 1] * dp[2 * k + 1]);
          asm volatile("" ::"v"(w[k]));   // keeps the pair in this slot
        }
    } else {
      const int ks = i - NX - KS;
      if (ks == 0) dp = dinit;
      dp = mfma32x32x16(frag[i], of[ks], dp);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  dsn[0] = as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
  dsn[1] = as_bf16x8(make_uint4(w[4], w[5], w[6], w[7]));
}

}  // namespace

template <int D>
__global__ __launch_bounds__(512, 1) void dq_partials_bf16(
    Geom g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_p,
    const uint16_t* __restrict__ v_p, const uint16_t* __restrict__ k_r,
    const uint16_t* __restrict__ v_r, const uint16_t* __restrict__ d_o,
    const float* __restrict__ lse, const float* __restrict__ Dvec, float* __restrict__ dq_part) {
  using C = DqRingCfg<D>;
  constexpr int KS = C::KS, DT = C::DT;
  // K tiles of the four stages first, then the V tiles (above 64 KiB, read through
  // biased offsets).
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
  // workgroup, [n_full, n_sub) is masked.
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
  FarFrags<D> far;
  far.template init<true, false>(fr);

  auto issue_stage = [&](int b, int st) {
    const int64_t off = (int64_t)st * C::BN * sbytes;
    const int rows = n_keys - st * C::BN;
    dl.issue(lds_addr(KT[b]), reinterpret_cast<const char*>(kc) + off, rows, (uint32_t)sbytes);
    dl.issue(lds_addr(VT[b]), reinterpret_cast<const char*>(vc) + off, rows, (uint32_t)sbytes);
  };
  auto issue_any = [&](int st) {
    switch (st & 3) {
      case 0: issue_stage(0, st); break;
      case 1: issue_stage(1, st); break;
      case 2: issue_stage(2, st); break;
      default: issue_stage(3, st); break;
    }
  };
  // Entering stage st: its loads are done (only stage st+1's may still be in flight),
  // every wave is past its reads of stage st-2's buffer, and stage st+2 is loaded into it.
  int entered = -1;
  auto enter_stage = [&](int st) {
    if (st + 1 < n_stages) wait_vmcnt_n<C::LOADS>(); else wait_vmcnt0();
    __syncthreads();
    if (st + 2 < n_stages) issue_any(st + 2);
    entered = st;
  };
  if (n_stages > 0) issue_any(0);
  if (n_stages > 1) issue_any(1);

  const int m = w.m0 + wave * 32 + col;
  const int r = m / g.grp, h = w.g * g.grp + m % g.grp;
  const bool valid = m < m_hi && r < rl;
  const int lim = resp ? min(r, n_keys - 1) : n_keys - 1;
  const int64_t row = ((int64_t)w.k * g.R + r) * g.Hq + h;
  const int64_t orow = m < m_hi ? ((int64_t)w.part * g.part_step + row * g.row_step) : -1;
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
  int wmax = lim;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) wmax = max(wmax, __shfl_xor(wmax, off, 64));

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.0f;
  const float c2 = g.c2;

  if (n_keys > 0) enter_stage(0);

  if (n_full > 0) {
    f32x16 s, dp;
    dqr_scores<D>(fr, far, KT[0], VT[0], 0, qf, of, dinit, s, dp);   // S(0), dP(0)
    bf16x8 dsp[2];                                                    // dS(u-1)

    // Block B(u), u = J mod 8: dQ(u-1) with the vector work of u, then S, dP of u+1;
    // compile-time buffers.  The last block also computes S, dP of subtile n_full, which
    // are never used (the masked path recomputes them) and read a buffer with no loads
    // in flight.
    auto block = [&](auto jc, auto pc, int u) {
      constexpr int J = decltype(jc)::value;
      constexpr bool PREV = decltype(pc)::value;
      constexpr int SX = ((J + 7) >> 1) & 3, SUBX = (J + 7) & 1;   // subtile u-1
      constexpr int SY = ((J + 1) >> 1) & 3, SUBY = (J + 1) & 1;   // subtile u+1
      constexpr int SN = (SY + 2) & 3;                              // stage (u+1)/2 + 2's buffer
      if (J & 1) {   // subtile u+1 starts stage (u+1)/2
        const int st = (u + 1) >> 1;
        if (st + 1 < n_stages) wait_vmcnt_n<C::LOADS>(); else wait_vmcnt0();
        __syncthreads();
        if (st + 2 < n_stages) issue_stage(SN, st + 2);
        entered = st;
      }
      bf16x8 dsn[2];
      dqr_block_body<D, PREV>(fr, far, KT[SX], SUBX, KT[SY], VT[SY], SUBY, qf, of, dinit, c2, lse2, dsp, acc,
                              s, dp, dsn);
      // dS(u) must be formed in this block, not sunk toward its use in the next one
      pin_operands(dsn, lse2);
      dsp[0] = dsn[0];
      dsp[1] = dsn[1];
    };
    using T = std::true_type;
    using F = std::false_type;
    block(std::integral_constant<int, 0>{}, F{}, 0);
    int u = 1;
    // straight-line groups of eight blocks (u = 8i+1 .. 8i+8): every block's buffers are
    // compile-time
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
    // dQ of the last pipelined subtile
    const int ul = n_full - 1;
    const int bl = (ul >> 1) & 3;
    dqr_dq<D>(fr, bl == 0 ? kt0 : bl == 1 ? kt1 : bl == 2 ? kt2 : kt3, ul & 1, dsp, acc);
  }

  // Masked subtiles near the causal diagonal or a chunk end.
  for (int u = n_full; u < n_sub; ++u) {
    const int st = u >> 1;
    while (entered < st) enter_stage(entered + 1);
    const int rel = u * 32;
    if (rel > wmax) continue;
    const int b = st & 3;
    const char* const kt = b == 0 ? kt0 : b == 1 ? kt1 : b == 2 ? kt2 : kt3;
    const char* const vt = b == 0 ? vt0 : b == 1 ? vt1 : b == 2 ? vt2 : vt3;
    f32x16 s, dp;
    dqr_scores<D>(fr, far, kt, vt, u & 1, qf, of, dinit, s, dp);
    uint32_t wv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float e[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int i = 2 * k + x;
        const int key = rel + (i >> 2) * 8 + hl * 4 + (i & 3);
        const float p = key > lim ? 0.0f : fast_exp2(fmaf(s[i], c2, -lse2));
        e[x] = p * dp[i];
      }
      wv[k] = pack_bf16x2(e[0], e[1]);
    }
    bf16x8 dsf[2];
    dsf[0] = as_bf16x8(make_uint4(wv[0], wv[1], wv[2], wv[3]));
    dsf[1] = as_bf16x8(make_uint4(wv[4], wv[5], wv[6], wv[7]));
    dqr_dq<D>(fr, kt, u & 1, dsf, acc);
  }
  // The direct loads are not tracked by the compiler: none may still be writing LDS when
  // the workgroup ends (every issued stage has been entered and waited for by now; this
  // makes it unconditional).
  wait_vmcnt0();

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

hipError_t launch_dq_partials_bf16(const Geom& g, const AttnPtrs& a, hipStream_t s) {
  const int64_t n = tile_work_count(g, DqRingCfg<128>::BM);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)xcd_grid(n)), block(64 * DqRingCfg<128>::WAVES);
  const uint16_t *q = (const uint16_t*)a.q, *kp = (const uint16_t*)a.k_p, *vp = (const uint16_t*)a.v_p;
  const uint16_t *kr = (const uint16_t*)a.k_r, *vr = (const uint16_t*)a.v_r, *dO = (const uint16_t*)a.d_o;
  if (g.dqk == 64)
    hipLaunchKernelGGL(dq_partials_bf16<64>, grid, block, 0, s, g, q, kp, vp, kr, vr, dO, a.lse, a.Dvec, a.dq_part);
  else
    hipLaunchKernelGGL(dq_partials_bf16<128>, grid, block, 0, s, g, q, kp, vp, kr, vr, dO, a.lse, a.Dvec, a.dq_part);
  return hipGetLastError();
}

}  // namespace rr
