// Key-parallel K/V gradients over a packed row stream (gfx950): the response's own dK_r,
// dV_r of the reverse block walk, and the resident prompt's dK_p, dV_p of the
// full-sequence differential mode.
//
// Sources: ai.thesatyajit.com/articles/longstraw-2m-rl, section "The move: change the
// graph boundary" (the full-sequence gradient is the direct response term plus a term
// that flows back through the prompt state; the response-only contract keeps the first
// and drops the second) and section "Two incompatible architectures, same transaction"
// (response blocks replayed in reverse); networkfinds.com/long-context-rl-is-a-state-
// lifetime-problem, section "Preserve gradient semantics, not just forward outputs"
// (differential validation against a conventional run).  The response-only backward
// calls only resp_dkdv_bf16; the prompt term is formed only when asked for.
//
// With the global statistics of row i (lse_i, and D_i = dO_i . O_i), for key j of KV head g
// and every row i of a query head of g that sees it:
//   p_ij = exp(tau q_i.k_j - lse_i),  ds_ij = p_ij (dO_i.v_j - D_i),
//   dK[j] = tau sum_i ds_ij q_i,      dV[j] = sum_i p_ij dO_i.
// Every row sees every prompt key; a response key j is seen by the rows i >= j of its
// own response.
//
// pg_pack: the launch's rows of KV head g, flattened per response (m = r * grp + hh) and
// padded with empty rows to a multiple of 64, become one contiguous stream per KV head: Q
// and dO rows, and per 64-row stage the rows' lse * log2(e) followed by their -D.  An empty
// row has lse = +inf and contributes p = 0.
//
// prompt_dkdv_bf16: one workgroup per (KV head, 128 prompt keys), four waves (one per SIMD)
// of 32 keys.  A wave keeps its keys' K and V rows in registers (the B operands of
// S = Q K^T and dP = dO V^T) and its dK^T, dV^T accumulators.  The stream's 64-row stages
// pass through a ring of four LDS buffers, loaded straight from global memory two stages
// ahead, one barrier per stage.  Per 32-row subtile u: S, and dP - D (the accumulation
// starts from -D); p = 2^(S c2 - lse2), dS = p (dP - D), both rounded to bf16;
// dV^T += dO^T P and dK^T += Q^T dS, with dO^T and Q^T read by transposing LDS reads in
// the row order of the score tile's C registers.  Block B(u) issues the dV/dK MFMAs of
// subtile u-1 and the S, dP MFMAs of u+1 while the vector ALUs form p and dS of u; it is
// laid out by hand in slots (each slot's LDS reads two slots ahead of its MFMA) separated
// by scheduling barriers.
//
// resp_dkdv_bf16: the same pipeline for a tile of one response's own keys, over that
// response's rows from the tile's first key on, in decreasing row order, cut into
// segments of stages so that the tiles' work items cost alike; the subtiles at the causal
// diagonal run unpipelined with the mask.  resp_dkdv_reduce adds the later segments'
// partial sums in segment order.
#include <type_traits>

#include "k_attn_tile.h"
#include "k_lds.h"
#include "k_ring.h"
#include "k_split.h"
#include "kernels.h"

namespace rr {

#ifndef RR_AHEAD
#define RR_AHEAD 2   // slots between a fragment's LDS read and its MFMA
#endif

namespace {

constexpr int kPgStage = kPgStageRows;

template <int D>
struct PgCfg {
  static constexpr int WAVES = 4;
  static constexpr int KEYS = 32 * WAVES;   // prompt keys per workgroup
  static constexpr int BM = kPgStage;
  static constexpr int KS = D / 16, DT = D / 32;
  static constexpr int TILE = BM * D * 2;   // bytes of one [BM][D] bf16 tile
  // direct loads per wave per stage: the Q and dO tiles, plus one for the statistics
  static constexpr int LOADS = 2 * (BM * D / 8) / (64 * WAVES) + 1;
  static_assert(LOADS < 16, "vmcnt field");
};

// ---- packing ------------------------------------------------------------------------------
// One wave per stream row n of KV head gh.
template <bool BF16, int D>
__global__ __launch_bounds__(256) void pg_pack(Geom g, PgGeom pg, const void* __restrict__ q,
                                               const float* __restrict__ o,
                                               const float* __restrict__ lse,
                                               const void* __restrict__ d_o, void* __restrict__ qs,
                                               void* __restrict__ os, float* __restrict__ sts) {
  constexpr int E = D / 64;   // elements per lane
  const int64_t wid = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (wid >= (int64_t)g.Hkv * pg.n_rows) return;
  const int gh = (int)(wid / pg.n_rows);
  const int n = (int)(wid % pg.n_rows);
  int k = 0;
  while (k + 1 < g.K && n >= pg.off[k + 1]) ++k;
  const int m = pg.m_lo + (n - pg.off[k]);   // flattened row r * grp + hh of response k
  const int r_hi = g.r_len[k] < g.row_hi ? g.r_len[k] : g.row_hi;
  const bool valid = m < r_hi * g.grp && m >= g.row_lo * g.grp;
  const int r = valid ? m / g.grp : 0, hh = valid ? m % g.grp : 0;
  const int64_t src = ((int64_t)k * g.R + r) * g.Hq + gh * g.grp + hh;
  const int64_t dst = (int64_t)gh * pg.n_rows + n;
  float dsum = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int c = lane * E + e;
    if (BF16) {
      const uint16_t* q16 = static_cast<const uint16_t*>(q);
      const uint16_t* o16 = static_cast<const uint16_t*>(d_o);
      const uint16_t qv = valid ? q16[src * D + c] : (uint16_t)0;
      const uint16_t ov = valid ? o16[src * D + c] : (uint16_t)0;
      static_cast<uint16_t*>(qs)[dst * D + c] = qv;
      static_cast<uint16_t*>(os)[dst * D + c] = ov;
      if (valid) dsum += bf16_bits_to_f32(ov) * o[src * D + c];
    } else {
      const float qv = valid ? static_cast<const float*>(q)[src * D + c] : 0.0f;
      const float ov = valid ? static_cast<const float*>(d_o)[src * D + c] : 0.0f;
      static_cast<float*>(qs)[dst * D + c] = qv;
      static_cast<float*>(os)[dst * D + c] = ov;
      if (valid) dsum += ov * o[src * D + c];
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) dsum += __shfl_xor(dsum, off, 64);
  if (lane == 0) {
    float* st = sts + ((int64_t)gh * (pg.n_rows / kPgStage) + n / kPgStage) * (2 * kPgStage);
    st[n % kPgStage] = valid ? lse[src] * kLog2e : INFINITY;
    st[kPgStage + n % kPgStage] = valid ? -dsum : 0.0f;
  }
}

// ---- bf16 MFMA kernel ---------------------------------------------------------------------

// lse2 and -D of the rows of subtile `sub` of a stage, in the row order of the C registers
// of a 32x32 score tile (register i holds row 8(i/4) + 4h + i%4).
__device__ __forceinline__ void pg_stats(const float* sb, int sub, float (&l2)[16], f32x16& ndv) {
  const int hl = (threadIdx.x >> 5) & 1;
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const float4 a = *reinterpret_cast<const float4*>(sb + 32 * sub + 8 * i4 + 4 * hl);
    const float4 b = *reinterpret_cast<const float4*>(sb + kPgStage + 32 * sub + 8 * i4 + 4 * hl);
    l2[4 * i4 + 0] = a.x;
    l2[4 * i4 + 1] = a.y;
    l2[4 * i4 + 2] = a.z;
    l2[4 * i4 + 3] = a.w;
    ndv[4 * i4 + 0] = b.x;
    ndv[4 * i4 + 1] = b.y;
    ndv[4 * i4 + 2] = b.z;
    ndv[4 * i4 + 3] = b.w;
  }
}

// S and dP - D of one subtile (unpipelined form).
template <int D>
__device__ __forceinline__ void pg_scores(const Frag<D>& fr, const FarFrags<D>& far, const char* Qt,
                                          const char* Ot, int sub, const bf16x8 (&kf)[D / 16],
                                          const bf16x8 (&vf)[D / 16], const f32x16& ndv, f32x16& s,
                                          f32x16& dp) {
#pragma unroll
  for (int i = 0; i < 16; ++i) s[i] = 0.0f;
  dp = ndv;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    s = mfma32x32x16(fr.row(Qt, sub, ks), kf[ks], s);
    dp = mfma32x32x16(far.row(Ot, sub, ks), vf[ks], dp);
  }
}

// dV^T += dO^T P and dK^T += Q^T dS of one subtile (unpipelined form).
template <int D>
__device__ __forceinline__ void pg_dkdv(const Frag<D>& fr, const FarFrags<D>& far, const char* Qt,
                                        const char* Ot, int sub, const bf16x8 (&pp)[2],
                                        const bf16x8 (&dsp)[2], f32x16 (&dk)[D / 32],
                                        f32x16 (&dv)[D / 32]) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      dv[dt] = mfma32x32x16(far.trans_frag(Ot, sub, h2, dt), pp[h2], dv[dt]);
      dk[dt] = mfma32x32x16(fr.trans_frag(Qt, sub, h2, dt), dsp[h2], dk[dt]);
    }
}

// One pipelined block.  With PREV the slots are: 2 D/16 dV, dK MFMAs of subtile u-1
// (transposed dO and Q fragments), carrying the exponentials of subtile u (each p
// replaces its S value) and the bf16 packing of P(u); D/16 S MFMAs of subtile u+1,
// carrying dS = p (dP - D) and its packing (dP(u) is still live there); D/16 dP MFMAs of
// subtile u+1, starting from -D of its rows.  Every slot first issues the LDS reads of
// the fragment two slots ahead.
template <int D, bool PREV>
__device__ __forceinline__ void pg_block_body(const Frag<D>& fr, const FarFrags<D>& far, const char* Qx,
                                              const char* Ox, int subx, const char* Qy, const char* Oy,
                                              int suby, const bf16x8 (&kf)[D / 16],
                                              const bf16x8 (&vf)[D / 16], float c2, const float (&l2)[16],
                                              const f32x16& ndv, const bf16x8 (&pp)[2],
                                              const bf16x8 (&dsp)[2], f32x16 (&dk)[D / 32],
                                              f32x16 (&dv)[D / 32], f32x16& s, f32x16& dp,
                                              bf16x8 (&pn)[2], bf16x8 (&dsn)[2]) {
  constexpr int KS = D / 16, DT = D / 32;
  constexpr int NX = PREV ? 4 * DT : 0;   // dV, dK slots
  constexpr int NSLOT = NX + 2 * KS;
  auto load = [&](int i) -> bf16x8 {
    if (i < NX) {
      const int j = i >> 1;   // (dt, h2) = (j >> 1, j & 1); even slots dV, odd slots dK
      return (i & 1) ? fr.trans_frag(Qx, subx, j & 1, j >> 1) : far.trans_frag(Ox, subx, j & 1, j >> 1);
    }
    const int j = i - NX;
    return j < KS ? fr.row(Qy, suby, j) : far.row(Oy, suby, j - KS);
  };
  float p[16];
  uint32_t wp[8], wd[8];
  if (!PREV) {
    // first block: no dV/dK MFMAs to overlap, so the exponentials and P run up front
#pragma unroll
    for (int e = 0; e < 16; ++e) p[e] = fast_exp2(fmaf(s[e], c2, -l2[e]));
#pragma unroll
    for (int k = 0; k < 8; ++k) wp[k] = pack_bf16x2(p[2 * k], p[2 * k + 1]);
    __builtin_amdgcn_sched_barrier(0);
  }
  bf16x8 frag[NSLOT];
#pragma unroll
  for (int i = 0; i < RR_AHEAD && i < NSLOT; ++i) frag[i] = load(i);
#pragma unroll
  for (int i = 0; i < NSLOT; ++i) {
    if (i + RR_AHEAD < NSLOT) frag[i + RR_AHEAD] = load(i + RR_AHEAD);
    if (i < NX) {
      const int j = i >> 1;
      if (i & 1)
        dk[j >> 1] = mfma32x32x16(frag[i], dsp[j & 1], dk[j >> 1]);
      else
        dv[j >> 1] = mfma32x32x16(frag[i], pp[j & 1], dv[j >> 1]);
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if ((e * NX) / 16 == i) {
          p[e] = fast_exp2(fmaf(s[e], c2, -l2[e]));
          asm volatile("" ::"v"(p[e]));   // keeps the exponential in this slot
        }
      // P pairs once both exponentials are two slots old
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (NX / 2 + (k * NX) / 16 == i) {
          wp[k] = pack_bf16x2(p[2 * k], p[2 * k + 1]);
          asm volatile("" ::"v"(wp[k]));
        }
    } else if (i < NX + KS) {
      const int ks = i - NX;
      if (ks == 0) {
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = 0.0f;
      }
      s = mfma32x32x16(frag[i], kf[ks], s);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if ((k * KS) / 8 == ks) {
          wd[k] = pack_bf16x2(p[2 * k] * dp[2 * k], p[2 * k + 1] * dp[2 * k + 1]);
          asm volatile("" ::"v"(wd[k]));   // keeps the pair in this slot
        }
    } else {
      const int ks = i - NX - KS;
      if (ks == 0) dp = ndv;
      dp = mfma32x32x16(frag[i], vf[ks], dp);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  pn[0] = as_bf16x8(make_uint4(wp[0], wp[1], wp[2], wp[3]));
  pn[1] = as_bf16x8(make_uint4(wp[4], wp[5], wp[6], wp[7]));
  dsn[0] = as_bf16x8(make_uint4(wd[0], wd[1], wd[2], wd[3]));
  dsn[1] = as_bf16x8(make_uint4(wd[4], wd[5], wd[6], wd[7]));
}

// Direct load of one stage's statistics (2 x 64 fp32 = 512 bytes): wave w loads half
// w & 1 (64 lanes x 4 bytes); waves 2 and 3 load the same bytes to the same place as
// waves 0 and 1, so every wave issues the same number of loads per stage.
__device__ __forceinline__ void pg_issue_stats(uint32_t tile_lds, const char* base) {
  const int lane = threadIdx.x & 63;
  const uint32_t half = (uint32_t)(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & 1) * 256u;
  const uint32_t lds = tile_lds + half;
  const uint32_t off = half + (uint32_t)lane * 4u;
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, %2"
      :
      : "s"(lds), "v"(off), "s"(base)
      : "memory", "m0");
}

}  // namespace

// Keys [key_lo, key_lo + n_keys) of the resident K/V; outputs indexed from key_lo.
template <int D>
__global__ __launch_bounds__(256, 1) void prompt_dkdv_bf16(
    PgGeom pg, int64_t key_lo, int64_t n_keys, int Hkv, float tau, float c2, const uint16_t* __restrict__ k_p,
    const uint16_t* __restrict__ v_p, const uint16_t* __restrict__ qs, const uint16_t* __restrict__ os,
    const float* __restrict__ sts, float* __restrict__ dk_p, float* __restrict__ dv_p, int accumulate) {
  using C = PgCfg<D>;
  constexpr int KS = C::KS, DT = C::DT;
  // One array, so the layout is fixed: the Q tiles of the four stages below 64 KiB (read
  // through plain offsets), then the dO tiles (read through biased offsets), then the
  // statistics.
  __shared__ __attribute__((aligned(1024))) char lds[8 * C::TILE + 4 * 2 * kPgStage * sizeof(float)];
  char* const QT[4] = {lds, lds + C::TILE, lds + 2 * C::TILE, lds + 3 * C::TILE};
  char* const OT[4] = {lds + 4 * C::TILE, lds + 5 * C::TILE, lds + 6 * C::TILE, lds + 7 * C::TILE};
  float* const st0 = reinterpret_cast<float*>(lds + 8 * C::TILE);
  float* const SB[4] = {st0, st0 + 2 * kPgStage, st0 + 4 * kPgStage, st0 + 6 * kPgStage};

  const int64_t n_kt = (n_keys + C::KEYS - 1) / C::KEYS;
  const int64_t idx = xcd_work_index((int64_t)Hkv * n_kt);
  if (idx < 0) return;
  const int64_t kt = idx % n_kt;
  const int gh = (int)(idx / n_kt);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hl = lane >> 5, col = lane & 31;
  const int64_t key = kt * C::KEYS + wave * 32 + col;   // relative to key_lo
  const bool kvalid = key < n_keys;

  // this wave's K and V rows (B operands): key `key`, dims 16 ks + 8 hl .. +8
  bf16x8 kf[KS], vf[KS];
  const int64_t kvrow = (key_lo + (kvalid ? key : 0)) * Hkv + gh;   // resident row
  const int64_t outrow = (kvalid ? key : 0) * Hkv + gh;             // output row
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kf[ks] = as_bf16x8(kvalid ? *reinterpret_cast<const uint4*>(k_p + kvrow * D + ks * 16 + hl * 8)
                              : make_uint4(0, 0, 0, 0));
    vf[ks] = as_bf16x8(kvalid ? *reinterpret_cast<const uint4*>(v_p + kvrow * D + ks * 16 + hl * 8)
                              : make_uint4(0, 0, 0, 0));
  }

  const int n_stages = pg.n_rows / C::BM;
  const int n_sub = 2 * n_stages;
  const char* const qb = reinterpret_cast<const char*>(qs + (int64_t)gh * pg.n_rows * D);
  const char* const ob = reinterpret_cast<const char*>(os + (int64_t)gh * pg.n_rows * D);
  const char* const sbase = reinterpret_cast<const char*>(sts + (int64_t)gh * n_stages * 2 * kPgStage);
  DirectLoadRows<D, C::BM, C::WAVES> dl;
  dl.init();
  Frag<D> fr;
  fr.init();
  FarFrags<D> far;
  far.template init<true, true>(fr);

  auto issue_stage = [&](int b, int st) {
    const int64_t off = (int64_t)st * C::TILE;
    dl.issue(lds_addr(QT[b]), qb + off, C::BM, (uint32_t)(D * 2));
    dl.issue(lds_addr(OT[b]), ob + off, C::BM, (uint32_t)(D * 2));
    pg_issue_stats(lds_addr(SB[b]), sbase + (int64_t)st * (2 * kPgStage * 4));
  };
  auto issue_any = [&](int st) {
    switch (st & 3) {
      case 0: issue_stage(0, st); break;
      case 1: issue_stage(1, st); break;
      case 2: issue_stage(2, st); break;
      default: issue_stage(3, st); break;
    }
  };

  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) dk[dt][i] = dv[dt][i] = 0.0f;

  if (n_stages > 0) {
    issue_any(0);
    if (n_stages > 1) issue_any(1);
    // entering stage 0: its loads are done (only stage 1's may still be in flight)
    if (n_stages > 1) wait_vmcnt_n<C::LOADS>(); else wait_vmcnt0();
    __syncthreads();
    if (n_stages > 2) issue_any(2);

    float l2[16];
    f32x16 ndv, s, dp;
    pg_stats(SB[0], 0, l2, ndv);
    pg_scores<D>(fr, far, QT[0], OT[0], 0, kf, vf, ndv, s, dp);   // S(0), dP(0)
    bf16x8 pp[2], dsp[2];                                          // P(u-1), dS(u-1)

    // Block B(u), u = J mod 8: dV/dK(u-1) with the vector work of u, then S, dP of u+1;
    // compile-time buffers.  The last block also forms S, dP of subtile n_sub, which are
    // never used and read a buffer with no loads in flight.
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
      }
      float l2n[16];
      f32x16 ndvn;
      pg_stats(SB[SY], SUBY, l2n, ndvn);
      bf16x8 pn[2], dsn[2];
      pg_block_body<D, PREV>(fr, far, QT[SX], OT[SX], SUBX, QT[SY], OT[SY], SUBY, kf, vf, c2, l2, ndvn, pp,
                             dsp, dk, dv, s, dp, pn, dsn);
      // P(u), dS(u) must be formed in this block, not sunk toward their use in the next one
      pin_operands(pn, c2);
      pin_operands(dsn, c2);
      pp[0] = pn[0];
      pp[1] = pn[1];
      dsp[0] = dsn[0];
      dsp[1] = dsn[1];
#pragma unroll
      for (int e = 0; e < 16; ++e) l2[e] = l2n[e];
    };
    using T = std::true_type;
    using F = std::false_type;
    block(std::integral_constant<int, 0>{}, F{}, 0);
    int u = 1;
    // straight-line groups of eight blocks (u = 8i+1 .. 8i+8): every block's buffers are
    // compile-time
    for (; u + 8 <= n_sub; u += 8) {
      block(std::integral_constant<int, 1>{}, T{}, u);
      block(std::integral_constant<int, 2>{}, T{}, u + 1);
      block(std::integral_constant<int, 3>{}, T{}, u + 2);
      block(std::integral_constant<int, 4>{}, T{}, u + 3);
      block(std::integral_constant<int, 5>{}, T{}, u + 4);
      block(std::integral_constant<int, 6>{}, T{}, u + 5);
      block(std::integral_constant<int, 7>{}, T{}, u + 6);
      block(std::integral_constant<int, 0>{}, T{}, u + 7);
    }
    if (u < n_sub) block(std::integral_constant<int, 1>{}, T{}, u++);
    if (u < n_sub) block(std::integral_constant<int, 2>{}, T{}, u++);
    if (u < n_sub) block(std::integral_constant<int, 3>{}, T{}, u++);
    if (u < n_sub) block(std::integral_constant<int, 4>{}, T{}, u++);
    if (u < n_sub) block(std::integral_constant<int, 5>{}, T{}, u++);
    if (u < n_sub) block(std::integral_constant<int, 6>{}, T{}, u++);
    if (u < n_sub) block(std::integral_constant<int, 7>{}, T{}, u++);
    // dV, dK of the last subtile
    const int ul = n_sub - 1;
    switch ((ul >> 1) & 3) {
      case 0: pg_dkdv<D>(fr, far, QT[0], OT[0], ul & 1, pp, dsp, dk, dv); break;
      case 1: pg_dkdv<D>(fr, far, QT[1], OT[1], ul & 1, pp, dsp, dk, dv); break;
      case 2: pg_dkdv<D>(fr, far, QT[2], OT[2], ul & 1, pp, dsp, dk, dv); break;
      default: pg_dkdv<D>(fr, far, QT[3], OT[3], ul & 1, pp, dsp, dk, dv); break;
    }
  }
  // The direct loads are not tracked by the compiler: none may still be writing LDS when
  // the workgroup ends.
  wait_vmcnt0();

  if (!kvalid) return;
  float* dkq = dk_p + outrow * D;
  float* dvq = dv_p + outrow * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = dt * 32 + i4 * 8 + hl * 4;
      float4 a = make_float4(dk[dt][4 * i4 + 0] * tau, dk[dt][4 * i4 + 1] * tau, dk[dt][4 * i4 + 2] * tau,
                             dk[dt][4 * i4 + 3] * tau);
      float4 b = make_float4(dv[dt][4 * i4 + 0], dv[dt][4 * i4 + 1], dv[dt][4 * i4 + 2], dv[dt][4 * i4 + 3]);
      if (accumulate) {
        const float4 a0 = *reinterpret_cast<const float4*>(dkq + d0);
        const float4 b0 = *reinterpret_cast<const float4*>(dvq + d0);
        a.x += a0.x;
        a.y += a0.y;
        a.z += a0.z;
        a.w += a0.w;
        b.x += b0.x;
        b.y += b0.y;
        b.z += b0.z;
        b.w += b0.w;
      }
      *reinterpret_cast<float4*>(dkq + d0) = a;
      *reinterpret_cast<float4*>(dvq + d0) = b;
    }
}

// ---- response keys: the causal dK_r, dV_r of the launch's rows ------------------------------
// A tile (response k, KV head g, 128 response keys j0 ..) sees the stream rows of response k
// with r >= j0 (the stream holds the launch's rows [row_lo, row_hi), so keys from row_hi on
// are untouched).  Its stages run from the response's last stream stage down to the one
// holding row j0, each stage's two subtiles upper first, so rows decrease along the
// sequence.  That run is cut into segments (k_split.h), one workgroup of four waves of 32
// keys each.  Within a segment, every subtile before n_full holds only rows r >= j0 + 127,
// which see every key of the tile (the pipelined blocks, as in the prompt kernel); the
// rest, near the causal diagonal (only in a tile's last segment), run unpipelined with
// p = 0 wherever key > row.  A tile's first segment adds its sums to dk_r, dv_r; a later
// one writes them to its partial slot, which resp_dkdv_reduce adds afterwards.
template <int D>
__global__ __launch_bounds__(256, 1) void resp_dkdv_bf16(
    Geom g, PgGeom pg, DkdvSplit sp, const uint16_t* __restrict__ k_r, const uint16_t* __restrict__ v_r,
    const uint16_t* __restrict__ qs, const uint16_t* __restrict__ os, const float* __restrict__ sts,
    float* __restrict__ slots, float* __restrict__ dk_r, float* __restrict__ dv_r) {
  using C = PgCfg<D>;
  constexpr int KS = C::KS, DT = C::DT;
  // the same fixed layout as prompt_dkdv_bf16
  __shared__ __attribute__((aligned(1024))) char lds[8 * C::TILE + 4 * 2 * kPgStage * sizeof(float)];
  char* const QT[4] = {lds, lds + C::TILE, lds + 2 * C::TILE, lds + 3 * C::TILE};
  char* const OT[4] = {lds + 4 * C::TILE, lds + 5 * C::TILE, lds + 6 * C::TILE, lds + 7 * C::TILE};
  float* const st0 = reinterpret_cast<float*>(lds + 8 * C::TILE);
  float* const SB[4] = {st0, st0 + 2 * kPgStage, st0 + 4 * kPgStage, st0 + 6 * kPgStage};

  static_assert(C::KEYS == kRespKeys, "tile width");
  // work item: (k, KV head, tile, segment); plain block order, so every XCD receives a mix
  // of tiles
  const DkdvItem item = dkdv_item(g, pg, sp, (int)blockIdx.x);
  if (item.k < 0) return;
  const int k = item.k, gh = item.gh, kt = item.kt;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hl = lane >> 5, col = lane & 31;
  const int kmax = g.r_len[k] < g.row_hi ? g.r_len[k] : g.row_hi;   // keys the rows can see
  const int j0 = kt * C::KEYS;
  const int key = j0 + wave * 32 + col;
  const bool kvalid = key < kmax;
  const int64_t kvrow = ((int64_t)k * g.R + (kvalid ? key : 0)) * g.Hkv + gh;
  bf16x8 kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kf[ks] = as_bf16x8(kvalid ? *reinterpret_cast<const uint4*>(k_r + kvrow * D + ks * 16 + hl * 8)
                              : make_uint4(0, 0, 0, 0));
    vf[ks] = as_bf16x8(kvalid ? *reinterpret_cast<const uint4*>(v_r + kvrow * D + ks * 16 + hl * 8)
                              : make_uint4(0, 0, 0, 0));
  }

  // stream stages of response k: stage s holds flattened rows m_lo + 64 s ..; this item
  // runs the segment's stages from stream stage n_top - 1 down
  const int grp = g.grp;
  const int n_stages = item.n_stages;
  const int n_top = item.n_top;
  const int n_sub = 2 * n_stages;
  // subtile u of the sequence: stage n_top - 1 - u / 2, upper half first; its first row is
  // m = m_lo + 64 n_top - 32 (u + 1)
  const int m_top = pg.m_lo + C::BM * n_top;
  const int n_full_raw = (m_top - (j0 + C::KEYS - 1) * grp) / 32;
  const int n_full = n_full_raw < 0 ? 0 : (n_full_raw > n_sub ? n_sub : n_full_raw);
  const int64_t row0 = (int64_t)gh * pg.n_rows + pg.off[k];
  const char* const qb = reinterpret_cast<const char*>(qs + row0 * D);
  const char* const ob = reinterpret_cast<const char*>(os + row0 * D);
  const char* const sbase =
      reinterpret_cast<const char*>(sts + ((int64_t)gh * (pg.n_rows / C::BM) + pg.off[k] / C::BM) * 2 * kPgStage);
  DirectLoadRows<D, C::BM, C::WAVES> dl;
  dl.init();
  Frag<D> fr;
  fr.init();
  FarFrags<D> far;
  far.template init<true, true>(fr);

  // sequence stage t is stream stage n_top - 1 - t
  auto issue_stage = [&](int b, int t) {
    const int st = n_top - 1 - t;
    const int64_t off = (int64_t)st * C::TILE;
    dl.issue(lds_addr(QT[b]), qb + off, C::BM, (uint32_t)(D * 2));
    dl.issue(lds_addr(OT[b]), ob + off, C::BM, (uint32_t)(D * 2));
    pg_issue_stats(lds_addr(SB[b]), sbase + (int64_t)st * (2 * kPgStage * 4));
  };
  auto issue_any = [&](int t) {
    switch (t & 3) {
      case 0: issue_stage(0, t); break;
      case 1: issue_stage(1, t); break;
      case 2: issue_stage(2, t); break;
      default: issue_stage(3, t); break;
    }
  };
  int entered = -1;
  auto enter_stage = [&](int t) {
    if (t + 1 < n_stages) wait_vmcnt_n<C::LOADS>(); else wait_vmcnt0();
    __syncthreads();
    if (t + 2 < n_stages) issue_any(t + 2);
    entered = t;
  };

  f32x16 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) dk[dt][i] = dv[dt][i] = 0.0f;
  const float c2 = g.c2;

  if (n_stages > 0) {
    issue_any(0);
    if (n_stages > 1) issue_any(1);
    enter_stage(0);
  }

  if (n_full > 0) {
    float l2[16];
    f32x16 ndv, s, dp;
    pg_stats(SB[0], 1, l2, ndv);
    pg_scores<D>(fr, far, QT[0], OT[0], 1, kf, vf, ndv, s, dp);   // subtile 0: stage 0, upper half
    bf16x8 pp[2], dsp[2];

    // Block B(u), u = J mod 8 (as in the prompt kernel, with the halves of a stage in
    // upper-first order).  The last block also forms S, dP of subtile n_full, never used.
    auto block = [&](auto jc, auto pc, int u) {
      constexpr int J = decltype(jc)::value;
      constexpr bool PREV = decltype(pc)::value;
      constexpr int SX = ((J + 7) >> 1) & 3, SUBX = 1 - ((J + 7) & 1);   // subtile u-1
      constexpr int SY = ((J + 1) >> 1) & 3, SUBY = 1 - ((J + 1) & 1);   // subtile u+1
      constexpr int SN = (SY + 2) & 3;
      if (J & 1) {   // subtile u+1 starts sequence stage (u+1)/2
        const int t = (u + 1) >> 1;
        if (t + 1 < n_stages) wait_vmcnt_n<C::LOADS>(); else wait_vmcnt0();
        __syncthreads();
        if (t + 2 < n_stages) issue_stage(SN, t + 2);
        entered = t;
      }
      float l2n[16];
      f32x16 ndvn;
      pg_stats(SB[SY], SUBY, l2n, ndvn);
      bf16x8 pn[2], dsn[2];
      pg_block_body<D, PREV>(fr, far, QT[SX], OT[SX], SUBX, QT[SY], OT[SY], SUBY, kf, vf, c2, l2, ndvn, pp,
                             dsp, dk, dv, s, dp, pn, dsn);
      pin_operands(pn, c2);
      pin_operands(dsn, c2);
      pp[0] = pn[0];
      pp[1] = pn[1];
      dsp[0] = dsn[0];
      dsp[1] = dsn[1];
#pragma unroll
      for (int e = 0; e < 16; ++e) l2[e] = l2n[e];
    };
    using T = std::true_type;
    using F = std::false_type;
    block(std::integral_constant<int, 0>{}, F{}, 0);
    int u = 1;
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
    const int ul = n_full - 1;
    const int subl = 1 - (ul & 1);
    switch ((ul >> 1) & 3) {
      case 0: pg_dkdv<D>(fr, far, QT[0], OT[0], subl, pp, dsp, dk, dv); break;
      case 1: pg_dkdv<D>(fr, far, QT[1], OT[1], subl, pp, dsp, dk, dv); break;
      case 2: pg_dkdv<D>(fr, far, QT[2], OT[2], subl, pp, dsp, dk, dv); break;
      default: pg_dkdv<D>(fr, far, QT[3], OT[3], subl, pp, dsp, dk, dv); break;
    }
  }

  // Subtiles near the causal diagonal: p = 0 wherever key > row.
  const float inv_grp = 1.0f / (float)grp;
  for (int u = n_full; u < n_sub; ++u) {
    const int t = u >> 1;
    while (entered < t) enter_stage(entered + 1);
    const int b = t & 3;
    const int sub = 1 - (u & 1);
    const int m_first = m_top - 32 * (u + 1);   // first flattened row of the subtile
    const char* const qt = lds + b * C::TILE;
    const char* const ot = lds + (4 + b) * C::TILE;
    const float* const sb = st0 + 2 * kPgStage * b;
    float l2[16];
    f32x16 ndv, s, dp;
    pg_stats(sb, sub, l2, ndv);
    pg_scores<D>(fr, far, qt, ot, sub, kf, vf, ndv, s, dp);
    uint32_t wp[8], wd[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      float pv[2], dsv[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int i = 2 * kk + x;
        const int m = m_first + (i >> 2) * 8 + hl * 4 + (i & 3);
        int r = (int)(((float)m + 0.5f) * inv_grp);   // m / grp; exact for m < 2^22
        r -= (r * grp > m) ? 1 : 0;
        r += ((r + 1) * grp <= m) ? 1 : 0;
        const float p = key > r ? 0.0f : fast_exp2(fmaf(s[i], c2, -l2[i]));
        pv[x] = p;
        dsv[x] = p * dp[i];
      }
      wp[kk] = pack_bf16x2(pv[0], pv[1]);
      wd[kk] = pack_bf16x2(dsv[0], dsv[1]);
    }
    bf16x8 pp[2], dsp[2];
    pp[0] = as_bf16x8(make_uint4(wp[0], wp[1], wp[2], wp[3]));
    pp[1] = as_bf16x8(make_uint4(wp[4], wp[5], wp[6], wp[7]));
    dsp[0] = as_bf16x8(make_uint4(wd[0], wd[1], wd[2], wd[3]));
    dsp[1] = as_bf16x8(make_uint4(wd[4], wd[5], wd[6], wd[7]));
    pg_dkdv<D>(fr, far, qt, ot, sub, pp, dsp, dk, dv);
  }
  // The direct loads are not tracked by the compiler: none may still be writing LDS when
  // the workgroup ends.
  wait_vmcnt0();

  if (!kvalid) return;
  if (item.slot >= 0) {
    // a later segment: its partial sums go to its slot, for the ordered reduction
    float* pk = slots + (item.slot * C::KEYS + wave * 32 + col) * (2 * D);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d0 = dt * 32 + i4 * 8 + hl * 4;
        *reinterpret_cast<float4*>(pk + d0) =
            make_float4(dk[dt][4 * i4 + 0], dk[dt][4 * i4 + 1], dk[dt][4 * i4 + 2], dk[dt][4 * i4 + 3]);
        *reinterpret_cast<float4*>(pk + D + d0) =
            make_float4(dv[dt][4 * i4 + 0], dv[dt][4 * i4 + 1], dv[dt][4 * i4 + 2], dv[dt][4 * i4 + 3]);
      }
    return;
  }
  float* dkq = dk_r + kvrow * D;
  float* dvq = dv_r + kvrow * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = dt * 32 + i4 * 8 + hl * 4;
      float4 a = *reinterpret_cast<const float4*>(dkq + d0);
      float4 b = *reinterpret_cast<const float4*>(dvq + d0);
      a.x += dk[dt][4 * i4 + 0] * g.tau;
      a.y += dk[dt][4 * i4 + 1] * g.tau;
      a.z += dk[dt][4 * i4 + 2] * g.tau;
      a.w += dk[dt][4 * i4 + 3] * g.tau;
      b.x += dv[dt][4 * i4 + 0];
      b.y += dv[dt][4 * i4 + 1];
      b.z += dv[dt][4 * i4 + 2];
      b.w += dv[dt][4 * i4 + 3];
      *reinterpret_cast<float4*>(dkq + d0) = a;
      *reinterpret_cast<float4*>(dvq + d0) = b;
    }
}

// Ordered reduction of the later segments: kDkdvReduceSplit workgroups per (k, KV head,
// tile) in item order, each over 128 / kDkdvReduceSplit of the tile's keys; for each valid
// key, dk_r += tau (slot_1 + slot_2 + ...) and dv_r += the same sum of the dV halves, the
// slots added in segment order.
constexpr int kDkdvReduceSplit = 16;

template <int D>
__global__ __launch_bounds__(256) void resp_dkdv_reduce(Geom g, PgGeom pg, DkdvSplit sp,
                                                        const float* __restrict__ slots, float* __restrict__ dk_r,
                                                        float* __restrict__ dv_r) {
  int idx = (int)(blockIdx.x / kDkdvReduceSplit);
  const int part = (int)(blockIdx.x % kDkdvReduceSplit);
  int k = 0;
  for (; k < g.K; ++k) {
    const int n = g.Hkv * resp_tiles(g, k);
    if (idx < n) break;
    idx -= n;
  }
  if (k >= g.K) return;
  const int nt = resp_tiles(g, k);
  const int gh = idx / nt, kt = idx % nt;
  const int n_items = resp_tile_items(g, pg, sp, k, kt);
  if (n_items < 2) return;
  const int64_t s0 = dkdv_tile_slot(g, pg, sp, k, gh, kt);
  const int kmax = g.r_len[k] < g.row_hi ? g.r_len[k] : g.row_hi;
  constexpr int V4 = 2 * D / 4;                           // float4 columns of a slot row (dK then dV)
  constexpr int KEYS = kRespKeys / kDkdvReduceSplit;      // keys of this workgroup
  for (int e = threadIdx.x; e < KEYS * V4; e += blockDim.x) {
    const int key_in = part * KEYS + e / V4, c = e % V4;
    const int key = kt * kRespKeys + key_in;
    if (key >= kmax) continue;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i = 0; i < n_items - 1; ++i) {
      const float4 b = *reinterpret_cast<const float4*>(slots + ((s0 + i) * kRespKeys + key_in) * (2 * D) + 4 * c);
      a.x += b.x;
      a.y += b.y;
      a.z += b.z;
      a.w += b.w;
    }
    const int64_t kvrow = ((int64_t)k * g.R + key) * g.Hkv + gh;
    const bool is_v = 4 * c >= D;
    float* dst = (is_v ? dv_r : dk_r) + kvrow * D + (4 * c - (is_v ? D : 0));
    const float sc = is_v ? 1.0f : g.tau;
    float4 o = *reinterpret_cast<const float4*>(dst);
    o.x += a.x * sc;
    o.y += a.y * sc;
    o.z += a.z * sc;
    o.w += a.w * sc;
    *reinterpret_cast<float4*>(dst) = o;
  }
}

// ---- fp32 kernel --------------------------------------------------------------------------
// Plain fp32 arithmetic for the fp32 configuration: a workgroup of 64 threads covers
// 64 / (D / 64) keys of one KV head, each key split over D / 64 threads (64 dims each, dot
// products combined across the halves).  Stream rows are staged 16 at a time in LDS.
template <int D>
__global__ __launch_bounds__(64) void prompt_dkdv_f32(PgGeom pg, int64_t key_lo, int64_t n_keys, int Hkv,
                                                      float tau, float c2,
                                                      const float* __restrict__ k_p,
                                                      const float* __restrict__ v_p,
                                                      const float* __restrict__ qs,
                                                      const float* __restrict__ os,
                                                      const float* __restrict__ sts,
                                                      float* __restrict__ dk_p, float* __restrict__ dv_p,
                                                      int accumulate) {
  constexpr int SPLIT = D / 64, KEYS = 64 / SPLIT, ROWS = 16;
  __shared__ float qrow[ROWS][D], orow[ROWS][D], l2s[ROWS], nds[ROWS];
  const int64_t n_kt = (n_keys + KEYS - 1) / KEYS;
  const int64_t kt = blockIdx.x % n_kt;
  const int gh = (int)(blockIdx.x / n_kt);
  const int t = threadIdx.x;
  const int part = t / KEYS;   // which 64 dims
  const int64_t key = kt * KEYS + t % KEYS;   // relative to key_lo
  const bool kvalid = key < n_keys;
  const int64_t kvrow = (key_lo + (kvalid ? key : 0)) * Hkv + gh;
  const int64_t outrow = (kvalid ? key : 0) * Hkv + gh;
  float kk[64], vv[64], dk[64], dv[64];
#pragma unroll
  for (int e = 0; e < 64; ++e) {
    kk[e] = kvalid ? k_p[kvrow * D + part * 64 + e] : 0.0f;
    vv[e] = kvalid ? v_p[kvrow * D + part * 64 + e] : 0.0f;
    dk[e] = dv[e] = 0.0f;
  }
  const float* qb = qs + (int64_t)gh * pg.n_rows * D;
  const float* ob = os + (int64_t)gh * pg.n_rows * D;
  const float* sb = sts + (int64_t)gh * (pg.n_rows / kPgStage) * 2 * kPgStage;
  for (int r0 = 0; r0 < pg.n_rows; r0 += ROWS) {
    for (int x = t; x < ROWS * D; x += 64) {
      qrow[x / D][x % D] = qb[(int64_t)r0 * D + x];
      orow[x / D][x % D] = ob[(int64_t)r0 * D + x];
    }
    if (t < ROWS) {
      const int n = r0 + t;
      const float* st = sb + (n / kPgStage) * 2 * kPgStage;
      l2s[t] = st[n % kPgStage];
      nds[t] = st[kPgStage + n % kPgStage];
    }
    __syncthreads();
    for (int rr = 0; rr < ROWS; ++rr) {
      float sdot = 0.0f, pdot = 0.0f;
#pragma unroll
      for (int e = 0; e < 64; ++e) {
        sdot = fmaf(qrow[rr][part * 64 + e], kk[e], sdot);
        pdot = fmaf(orow[rr][part * 64 + e], vv[e], pdot);
      }
      if (SPLIT == 2) {
        sdot += __shfl_xor(sdot, 32, 64);
        pdot += __shfl_xor(pdot, 32, 64);
      }
      const float p = fast_exp2(fmaf(sdot, c2, -l2s[rr]));
      const float ds = p * (pdot + nds[rr]);
#pragma unroll
      for (int e = 0; e < 64; ++e) {
        dk[e] = fmaf(ds, qrow[rr][part * 64 + e], dk[e]);
        dv[e] = fmaf(p, orow[rr][part * 64 + e], dv[e]);
      }
    }
    __syncthreads();
  }
  if (!kvalid) return;
#pragma unroll
  for (int e = 0; e < 64; ++e) {
    const int64_t at = outrow * D + part * 64 + e;
    const float a = dk[e] * tau, b = dv[e];
    dk_p[at] = accumulate ? dk_p[at] + a : a;
    dv_p[at] = accumulate ? dv_p[at] + b : b;
  }
}

// ---- launchers ----------------------------------------------------------------------------

hipError_t launch_pg_pack(const Geom& g, const PgGeom& pg, int dtype, const void* q, const float* o,
                          const float* lse, const void* d_o, void* qs, void* os, float* sts, hipStream_t s) {
  const int64_t waves = (int64_t)g.Hkv * pg.n_rows;
  if (waves == 0) return hipSuccess;
  const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  if (dtype == RR_BF16) {
    if (g.dqk == 64)
      hipLaunchKernelGGL((pg_pack<true, 64>), grid, block, 0, s, g, pg, q, o, lse, d_o, qs, os, sts);
    else
      hipLaunchKernelGGL((pg_pack<true, 128>), grid, block, 0, s, g, pg, q, o, lse, d_o, qs, os, sts);
  } else {
    if (g.dqk == 64)
      hipLaunchKernelGGL((pg_pack<false, 64>), grid, block, 0, s, g, pg, q, o, lse, d_o, qs, os, sts);
    else
      hipLaunchKernelGGL((pg_pack<false, 128>), grid, block, 0, s, g, pg, q, o, lse, d_o, qs, os, sts);
  }
  return hipGetLastError();
}

hipError_t launch_resp_dkdv(const Geom& g, const PgGeom& pg, const void* k_r, const void* v_r, const void* qs,
                            const void* os, const float* sts, float* slots, float* dk_r, float* dv_r,
                            hipStream_t s) {
  DkdvSplit sp{};
  int64_t n_slots = 0, tiles = 0;
  const int64_t items = plan_dkdv_split(g, pg, kDkdvItemsTarget, kDkdvMinSeg, sp, n_slots, tiles);
  if (items == 0) return hipSuccess;
  // a later segment of response k holds seg[k] stages, so response k has at most
  // total_k / seg[k] <= kDkdvItemsTarget of them
  if (n_slots > (int64_t)g.K * dkdv_slots_per_response(g.R, g.Hkv, g.grp)) return hipErrorInvalidValue;
  const uint16_t *kr = (const uint16_t*)k_r, *vr = (const uint16_t*)v_r;
  const uint16_t *q16 = (const uint16_t*)qs, *o16 = (const uint16_t*)os;
  if (g.dqk == 64)
    hipLaunchKernelGGL(resp_dkdv_bf16<64>, dim3((unsigned)items), dim3(256), 0, s, g, pg, sp, kr, vr, q16, o16, sts,
                       slots, dk_r, dv_r);
  else
    hipLaunchKernelGGL(resp_dkdv_bf16<128>, dim3((unsigned)items), dim3(256), 0, s, g, pg, sp, kr, vr, q16, o16,
                       sts, slots, dk_r, dv_r);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_slots == 0) return e;
  const dim3 rgrid((unsigned)(tiles * kDkdvReduceSplit));
  if (g.dqk == 64)
    hipLaunchKernelGGL(resp_dkdv_reduce<64>, rgrid, dim3(256), 0, s, g, pg, sp, slots, dk_r, dv_r);
  else
    hipLaunchKernelGGL(resp_dkdv_reduce<128>, rgrid, dim3(256), 0, s, g, pg, sp, slots, dk_r, dv_r);
  return hipGetLastError();
}

hipError_t launch_prompt_dkdv(const Geom& g, const PgGeom& pg, int dtype, const void* k_p, const void* v_p,
                              const void* qs, const void* os, const float* sts, int64_t key_lo, int64_t key_hi,
                              float* dk_p, float* dv_p, int accumulate, hipStream_t s) {
  const int64_t n_keys = key_hi - key_lo;
  if (n_keys <= 0) return hipSuccess;
  if (dtype == RR_BF16) {
    const int64_t n = (int64_t)g.Hkv * ((n_keys + PgCfg<128>::KEYS - 1) / PgCfg<128>::KEYS);
    const dim3 grid((unsigned)xcd_grid(n)), block(64 * PgCfg<128>::WAVES);
    const uint16_t *kp = (const uint16_t*)k_p, *vp = (const uint16_t*)v_p;
    const uint16_t *q16 = (const uint16_t*)qs, *o16 = (const uint16_t*)os;
    if (g.dqk == 64)
      hipLaunchKernelGGL(prompt_dkdv_bf16<64>, grid, block, 0, s, pg, key_lo, n_keys, g.Hkv, g.tau, g.c2, kp, vp,
                         q16, o16, sts, dk_p, dv_p, accumulate);
    else
      hipLaunchKernelGGL(prompt_dkdv_bf16<128>, grid, block, 0, s, pg, key_lo, n_keys, g.Hkv, g.tau, g.c2, kp, vp,
                         q16, o16, sts, dk_p, dv_p, accumulate);
  } else {
    const float *kp = (const float*)k_p, *vp = (const float*)v_p;
    const float *q32 = (const float*)qs, *o32 = (const float*)os;
    if (g.dqk == 64) {
      const int64_t n = (int64_t)g.Hkv * ((n_keys + 63) / 64);
      hipLaunchKernelGGL(prompt_dkdv_f32<64>, dim3((unsigned)n), dim3(64), 0, s, pg, key_lo, n_keys, g.Hkv, g.tau,
                         g.c2, kp, vp, q32, o32, sts, dk_p, dv_p, accumulate);
    } else {
      const int64_t n = (int64_t)g.Hkv * ((n_keys + 31) / 32);
      hipLaunchKernelGGL(prompt_dkdv_f32<128>, dim3((unsigned)n), dim3(64), 0, s, pg, key_lo, n_keys, g.Hkv, g.tau,
                         g.c2, kp, vp, q32, o32, sts, dk_p, dv_p, accumulate);
    }
  }
  return hipGetLastError();
}

}  // namespace rr
