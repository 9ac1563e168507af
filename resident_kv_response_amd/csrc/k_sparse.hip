// Latent-page sparse attention on MFMA (gfx950).
//
// Source: ai.thesatyajit.com/articles/longstraw-2m-rl, section "Two incompatible
// architectures, same transaction" (GLM instantiation): resident MLA latent pages of
// 512 + 64 dims, every head reading the same latent row, attention over the sparse
// selection of prompt positions plus the response's own causal rows, and the
// response-only backward.  Key = the whole 576-wide latent row, value = its first 512
// dims; 64 query heads share each row.
//
// sparse_fwd: one workgroup (8 waves) per query row, both 32-head tiles sharing each
// gathered tile.  Keys are the row's top-k prompt rows followed by response rows 0..i,
// gathered 32 at a time straight into LDS.  Wave w
// contracts dims [144w, 144w + 144) of the scores for all 64 heads; the four partial
// score tiles are exchanged through LDS and summed in a fixed order, so every wave holds
// the same scores and runs the same online softmax; wave w then accumulates the output
// for value dims [128w, 128w + 128).
//
// sparse_dq: the same structure for the backward: partial scores and partial dP = dO V^T
// (wave w: value dims [128w, 128w+128)), exchanged and summed; dS = P (dP - D); dQ^T for
// the wave's share of the 18 32-wide dim tiles.  For response keys it also writes P and
// dS (bf16) of every (row, head, key) pair, from which xty_gemm forms dK_r and dV_r.
//
// xty_gemm / xty_reduce: C[j][d] += alpha sum_{(i,h): i >= j} X[i][h][j] Y[i][h][d], the
// response-key gradients dK_r = tau dS^T Q and dV_r = P^T dO, with both operands read by
// transposing LDS reads from row-major tiles loaded straight into LDS.  The rows are split
// into chunks (one workgroup per chunk, key tile and dim tile) and the chunk partials are
// added in chunk order, so the sums are deterministic.
#include "k_lds.h"
#include "k_ring.h"
#include "kernels.h"

namespace rr {

constexpr int kLatD = 576, kLatDV = 512, kLatH = 64;

// Latent tile: rows of 576 bf16 (72 granules); logical granule g of row r stored at
// (g & ~7) | ((g & 7) ^ f(r)).  f(r) = ((r >> 1) & 1) << 2 | ((r >> 2) & 3) makes the 16
// consecutive rows of a row-fragment read and the 4 rows x 4 granules of a half-wave
// transposing read land on distinct banks (a row is 1152 bytes, so even and odd rows
// occupy different bank halves).
struct Lat {
  static constexpr int G = 72, ROW = 1152;
  static __device__ __forceinline__ int f(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
  static __device__ __forceinline__ int phys(int g, int r) { return (g & ~7) | ((g & 7) ^ f(r)); }
  static __device__ __forceinline__ int off(int r, int g) { return r * ROW + (phys(g, r) << 4); }
};
constexpr int kLatKeys = 32;
constexpr int kLatTile = kLatKeys * Lat::ROW;        // 36,864 bytes
constexpr int kLatInstr = kLatKeys * Lat::G / 64;    // 36 wave-wide loads per tile
constexpr int kLatSelMax = 4096;                     // largest top-k the kernels stage in LDS

// Gather keys [t0, t0 + 32) of a row's key list into `tile`: key t < n_sel is prompt row
// sel[t], key t >= n_sel is response row t - n_sel; keys at or past n_keys are
// redirected to key n_keys - 1 (masked by the caller).  `sel` is the row's selection in
// LDS, already clamped into [0, P): reading it there keeps the gathers free of waits on
// global loads (vmcnt drains in issue order, so waiting on a global index load would
// also wait on every gather in flight).  The 36 wave-wide loads are dealt over NW waves.
template <int NW = 4>
__device__ __forceinline__ void gather_tile(char* tile, const uint16_t* latent_p,
                                            const uint16_t* latent_rk, const int32_t* sel,
                                            int n_sel, int n_keys, int t0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int u = 0; u < (kLatInstr + NW - 1) / NW; ++u) {
    const int n = u * NW + wave;           // wave-wide load n fills LDS bytes [1024 n, 1024 n + 1024)
    if (kLatInstr % NW != 0 && n >= kLatInstr) break;
    const int p = 64 * n + lane;
    const int r = p / Lat::G, ph = p % Lat::G;
    const int g = (ph & ~7) | ((ph & 7) ^ Lat::f(r));
    const int t = min(t0 + r, n_keys - 1);
    const uint16_t* rowp = t < n_sel ? latent_p + (int64_t)sel[t] * kLatD : latent_rk + (int64_t)(t - n_sel) * kLatD;
    __builtin_amdgcn_global_load_lds(rowp + g * 8, (lds_void*)(tile + n * 1024), 16, 0, 0);
  }
}

// The row's selected positions, clamped into [0, P) so that a corrupt index list cannot
// address memory outside the resident pages, staged in LDS (ends with a barrier).
__device__ __forceinline__ void stage_selection(int32_t* sel_lds, const int32_t* sel, int n_sel, int64_t P) {
  for (int t = threadIdx.x; t < n_sel; t += blockDim.x) {
    const int64_t v = sel[t];
    sel_lds[t] = (int32_t)(v < 0 ? 0 : (v >= P ? P - 1 : v));
  }
  __syncthreads();
}

// Row fragment of a latent tile: A[m][k] = T[l%32][16*ks + 8h .. +8].
__device__ __forceinline__ bf16x8 lat_row(const char* tile, int ks) {
  const int lane = threadIdx.x & 63;
  return *reinterpret_cast<const bf16x8*>(tile + Lat::off(lane & 31, 2 * ks + (lane >> 5)));
}

// Transposed fragment of a latent tile: A[m][k] = T[row(k)][col0 + l%32], k-slots
// 0..3 <- rows 16*h2 + 4h + 0..3, 4..7 <- rows 16*h2 + 8 + 4h + 0..3 (the MFMA C layout's
// key order).
__device__ __forceinline__ bf16x8 lat_trans(const char* tile, int h2, int col0) {
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, grp = lane >> 4, h = lane >> 5;
  const int r = 16 * h2 + 4 * h + (i >> 2);
  const int c = col0 + 16 * (grp & 1) + 4 * (i & 3);
  const int within = (c & 7) * 2;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + Lat::off(r, c >> 3) + within));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + Lat::off(r + 8, c >> 3) + within));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Exchange of per-wave partial 32x32 tiles: xch[w][j][lane] holds registers 4j..4j+3 of
// lane `lane` of wave w.
struct Xch {
  float4 v[4][4][64];
};

__device__ __forceinline__ void xch_put(Xch& x, const f32x16& p, int slot) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < 4; ++j) x.v[slot][j][lane] = make_float4(p[4 * j], p[4 * j + 1], p[4 * j + 2], p[4 * j + 3]);
}

// Sum of the four partials in wave order (identical in every wave).
__device__ __forceinline__ void xch_sum(const Xch& x, f32x16& s) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float4 a = x.v[0][j][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const float4 b = x.v[w][j][lane];
      a.x += b.x;
      a.y += b.y;
      a.z += b.z;
      a.w += b.w;
    }
    s[4 * j] = a.x;
    s[4 * j + 1] = a.y;
    s[4 * j + 2] = a.z;
    s[4 * j + 3] = a.w;
  }
}

constexpr float kLatRescale = 8.0f;

// One workgroup = one query row and HT tiles of 32 heads, 4 waves per head tile (wave w:
// head tile w / 4, dim slice w % 4).  With HT = 2 both head tiles share each gathered tile;
// with HT = 1, blockIdx.x = 2 * row + tile.
template <int HT>
__global__ __launch_bounds__(256 * HT, 1) void sparse_fwd(Geom g, int topk, const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ latent_p,
                                                          const uint16_t* __restrict__ latent_r,
                                                          const int32_t* __restrict__ sel_idx,
                                                          float* __restrict__ o, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(1024))) char kv0[kLatTile];
  __shared__ __attribute__((aligned(1024))) char kv1[kLatTile];
  __shared__ __attribute__((aligned(16))) Xch xch[HT];
  __shared__ int32_t sel_lds[kLatSelMax];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int row = HT == 2 ? (int)blockIdx.x : (int)(blockIdx.x >> 1);
  const int ht = HT == 2 ? wv >> 2 : (int)(blockIdx.x & 1);
  const int wave = wv & 3;                                // dim slice within the head tile
  const int k = row / g.R, i = row % g.R;
  if (k >= g.K || i < g.row_lo || i >= g.row_hi) return;
  const int hl = lane >> 5, col = lane & 31;
  const int64_t hrow0 = (int64_t)row * kLatH + 32 * ht;   // (k, i, first head of the tile)
  if (i >= g.r_len[k]) {
    const int64_t h0 = (int64_t)row * kLatH + (HT == 2 ? 0 : 32 * ht);
    for (int e = threadIdx.x; e < 32 * HT * kLatDV; e += 256 * HT) o[h0 * kLatDV + e] = 0.0f;
    if (threadIdx.x < 32 * HT) lse[h0 + threadIdx.x] = -INFINITY;
    return;
  }
  const int n_keys = topk + i + 1;
  const int n_tiles = (n_keys + kLatKeys - 1) / kLatKeys;
  const uint16_t* latent_rk = latent_r + (int64_t)k * g.R * kLatD;
  stage_selection(sel_lds, sel_idx + (int64_t)row * topk, topk, g.P);
  const int32_t* sel = sel_lds;
  gather_tile<4 * HT>(kv0, latent_p, latent_rk, sel, topk, n_keys, 0);

  // Q fragments of this wave's 9 k-steps of the score contraction
  bf16x8 qf[9];
  const uint16_t* qrow = q + (hrow0 + col) * kLatD;
#pragma unroll
  for (int s = 0; s < 9; ++s)
    qf[s] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + 16 * (9 * wave + s) + 8 * hl));
  f32x16 acc[4];
  float m_run = kNegBig, l_run = 0.0f;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[dt][e] = 0.0f;

  auto tile_step = [&](const char* cur, char* nxt, int t) {
    wait_vmcnt0();
    __syncthreads();
    if (t + 1 < n_tiles) gather_tile<4 * HT>(nxt, latent_p, latent_rk, sel, topk, n_keys, (t + 1) * kLatKeys);
    // two independent accumulation chains (even and odd k-steps), each fragment read one
    // MFMA ahead, so the matrix core does not wait on a dependent result or a LDS read
    f32x16 sp, sq;
#pragma unroll
    for (int e = 0; e < 16; ++e) sp[e] = sq[e] = 0.0f;
    prio_mfma();
    {
      bf16x8 fcur = lat_row(cur, 9 * wave);
#pragma unroll
      for (int s = 0; s < 9; ++s) {
        const bf16x8 fnext = s + 1 < 9 ? lat_row(cur, 9 * wave + s + 1) : fcur;
        if (s & 1) sq = mfma32x32x16(fcur, qf[s], sq);
        else sp = mfma32x32x16(fcur, qf[s], sp);
        fcur = fnext;
      }
    }
    prio_valu();
#pragma unroll
    for (int e = 0; e < 16; ++e) sp[e] += sq[e];
    xch_put(xch[HT == 2 ? ht : 0], sp, wave);
    __syncthreads();
    f32x16 sc;
    xch_sum(xch[HT == 2 ? ht : 0], sc);
    const int rel = t * kLatKeys;
    if (rel + kLatKeys > n_keys) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = rel + (e >> 2) * 8 + hl * 4 + (e & 3);
        if (key >= n_keys) sc[e] = -INFINITY;
      }
    }
    float mx = sc[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sc[e]);
    mx = pair_max(mx);
    const float m_new = fmaxf(m_run, mx * g.c2);
    if (__any(m_new > m_run + kLatRescale)) {
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[dt][e] *= alpha;
      m_run = m_new;
    }
    float p[16], ls = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      p[e] = fast_exp2(fmaf(sc[e], g.c2, -m_run));
      ls += p[e];
    }
    l_run += ls;
    bf16x8 pf[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      uint4 uu;
      uu.x = pack_bf16x2(p[8 * h2 + 0], p[8 * h2 + 1]);
      uu.y = pack_bf16x2(p[8 * h2 + 2], p[8 * h2 + 3]);
      uu.z = pack_bf16x2(p[8 * h2 + 4], p[8 * h2 + 5]);
      uu.w = pack_bf16x2(p[8 * h2 + 6], p[8 * h2 + 7]);
      pf[h2] = as_bf16x8(uu);
    }
    prio_mfma();
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)       // four independent accumulators per k-step
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) acc[dt] = mfma32x32x16(lat_trans(cur, h2, 128 * wave + 32 * dt), pf[h2], acc[dt]);
    prio_valu();
  };
  for (int t = 0; t < n_tiles; t += 2) {
    tile_step(kv0, kv1, t);
    if (t + 1 < n_tiles) tile_step(kv1, kv0, t + 1);
  }

  const float l = pair_sum(l_run);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  float* dst = o + (hrow0 + col) * kLatDV + 128 * wave;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = 32 * dt + 8 * i4 + 4 * hl;
      *reinterpret_cast<float4*>(dst + d0) = make_float4(acc[dt][4 * i4] * inv, acc[dt][4 * i4 + 1] * inv,
                                                         acc[dt][4 * i4 + 2] * inv, acc[dt][4 * i4 + 3] * inv);
    }
  if (wave == 0 && hl == 0) lse[hrow0 + col] = l > 0.0f ? (m_run + log2f(l)) * kLn2 : -INFINITY;
}

// dQ of one query row and head tile, and the response pairs' P and dS.  pds layout:
// [K][R][64][R] bf16 (row, head, key); for row i the keys j in
// [0, min(R, round_up(i + 1, 128))) are written, zeros for j > i.
template <int HT>
__global__ __launch_bounds__(256 * HT, 1) void sparse_dq(Geom g, int topk, const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ latent_p,
                                                         const uint16_t* __restrict__ latent_r,
                                                         const int32_t* __restrict__ sel_idx,
                                                         const uint16_t* __restrict__ d_o,
                                                         const float* __restrict__ lse,
                                                         const float* __restrict__ Dvec,
                                                         float* __restrict__ dq, uint16_t* __restrict__ p_r,
                                                         uint16_t* __restrict__ ds_r, int accumulate) {
  __shared__ __attribute__((aligned(1024))) char kv0[kLatTile];
  __shared__ __attribute__((aligned(1024))) char kv1[kLatTile];
  __shared__ __attribute__((aligned(16))) Xch xs[HT];
  __shared__ __attribute__((aligned(16))) Xch xp[HT];
  __shared__ __attribute__((aligned(16))) uint2 dsx[HT][4][64];   // dS of the tile, bf16, by owner wave
  __shared__ int32_t sel_lds[kLatSelMax];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int row = HT == 2 ? (int)blockIdx.x : (int)(blockIdx.x >> 1);
  const int ht = HT == 2 ? wv >> 2 : (int)(blockIdx.x & 1);
  const int wave = wv & 3;                                // dim slice within the head tile
  const int xi = HT == 2 ? ht : 0;                        // this head tile's exchange buffers
  const int k = row / g.R, i = row % g.R;
  if (k >= g.K || i < g.row_lo || i >= g.row_hi) return;
  const int hl = lane >> 5, col = lane & 31;
  const int64_t hrow0 = (int64_t)row * kLatH + 32 * ht;
  const int64_t h0 = (int64_t)row * kLatH + (HT == 2 ? 0 : 32 * ht);   // first head of the workgroup
  if (i >= g.r_len[k]) {
    if (!accumulate)
      for (int e = threadIdx.x; e < 32 * HT * kLatD; e += 256 * HT) dq[h0 * kLatD + e] = 0.0f;
    return;
  }
  const int64_t pds_row = hrow0 * g.R;                // element offset of (k, i, first head, key 0)
  const int jz_end = min(g.R, ((i + 1 + 127) / 128) * 128);
  const int nz = jz_end - i - 1;                       // causal remainder of the last 128-key group
  for (int e = threadIdx.x; e < 32 * HT * nz; e += 256 * HT) {
    const int64_t at = h0 * g.R + (int64_t)(e / nz) * g.R + i + 1 + e % nz;
    p_r[at] = 0;
    ds_r[at] = 0;
  }
  const int n_keys = topk + i + 1;
  const int n_tiles = (n_keys + kLatKeys - 1) / kLatKeys;
  const uint16_t* latent_rk = latent_r + (int64_t)k * g.R * kLatD;
  stage_selection(sel_lds, sel_idx + (int64_t)row * topk, topk, g.P);
  const int32_t* sel = sel_lds;
  gather_tile<4 * HT>(kv0, latent_p, latent_rk, sel, topk, n_keys, 0);

  bf16x8 qf[9], of[8];
  const int64_t hr = hrow0 + col;
#pragma unroll
  for (int s = 0; s < 9; ++s)
    qf[s] = as_bf16x8(*reinterpret_cast<const uint4*>(q + hr * kLatD + 16 * (9 * wave + s) + 8 * hl));
#pragma unroll
  for (int s = 0; s < 8; ++s)
    of[s] = as_bf16x8(*reinterpret_cast<const uint4*>(d_o + hr * kLatDV + 16 * (8 * wave + s) + 8 * hl));
  const float lse2 = lse[hr] * kLog2e;
  const float dvv = Dvec[hr];
  // this wave's dQ dim tiles: 18 tiles of 32 split 5, 5, 4, 4
  const int dt_lo = wave < 2 ? 5 * wave : 10 + 4 * (wave - 2);
  const int n_dt = wave < 2 ? 5 : 4;
  f32x16 acc[5];
#pragma unroll
  for (int dt = 0; dt < 5; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[dt][e] = 0.0f;
  uint16_t* p_row = p_r + pds_row + (int64_t)col * g.R;
  uint16_t* ds_row = ds_r + pds_row + (int64_t)col * g.R;

  auto tile_step = [&](const char* cur, char* nxt, int t) {
    wait_vmcnt0();
    __syncthreads();
    if (t + 1 < n_tiles) gather_tile<4 * HT>(nxt, latent_p, latent_rk, sel, topk, n_keys, (t + 1) * kLatKeys);
    f32x16 sp, dpp;
#pragma unroll
    for (int e = 0; e < 16; ++e) sp[e] = dpp[e] = 0.0f;
    prio_mfma();
    {
      // the S and dP chains (score dims, value dims) alternate, so consecutive MFMAs are
      // independent
      bf16x8 fs = lat_row(cur, 9 * wave), fp = lat_row(cur, 8 * wave);
#pragma unroll
      for (int s = 0; s < 9; ++s) {
        const bf16x8 ns = s + 1 < 9 ? lat_row(cur, 9 * wave + s + 1) : fs;
        const bf16x8 np = s + 1 < 8 ? lat_row(cur, 8 * wave + s + 1) : fp;
        sp = mfma32x32x16(fs, qf[s], sp);
        if (s < 8) dpp = mfma32x32x16(fp, of[s], dpp);   // value dims
        fs = ns;
        fp = np;
      }
    }
    prio_valu();
    xch_put(xs[xi], sp, wave);
    xch_put(xp[xi], dpp, wave);
    __syncthreads();
    // This wave owns keys 8 wave + [0, 8) of the tile (C registers 4 wave .. 4 wave + 3 of
    // every lane): it sums the four partials of those entries in wave order, forms p and
    // dS = p (dP - D), shares dS in bf16, and writes the response pairs' P and dS.
    const int rel = t * kLatKeys;
    float4 sc = xs[xi].v[0][wave][lane], dp = xp[xi].v[0][wave][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const float4 a = xs[xi].v[w][wave][lane], b = xp[xi].v[w][wave][lane];
      sc.x += a.x;
      sc.y += a.y;
      sc.z += a.z;
      sc.w += a.w;
      dp.x += b.x;
      dp.y += b.y;
      dp.z += b.z;
      dp.w += b.w;
    }
    const int key0 = rel + 8 * wave + 4 * hl;          // 4 consecutive keys
    const float sv[4] = {sc.x, sc.y, sc.z, sc.w}, dv[4] = {dp.x, dp.y, dp.z, dp.w};
    float pe[4], de[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pe[e] = key0 + e < n_keys ? fast_exp2(fmaf(sv[e], g.c2, -lse2)) : 0.0f;
      de[e] = pe[e] * (dv[e] - dvv);
    }
    const uint2 dsw = make_uint2(pack_bf16x2(de[0], de[1]), pack_bf16x2(de[2], de[3]));
    dsx[xi][wave][lane] = dsw;
    if (key0 >= topk && key0 < n_keys) {              // response keys (keys past i: p = dS = 0)
      const int j = key0 - topk;
      *reinterpret_cast<uint2*>(p_row + j) = make_uint2(pack_bf16x2(pe[0], pe[1]), pack_bf16x2(pe[2], pe[3]));
      *reinterpret_cast<uint2*>(ds_row + j) = dsw;   // j + 3 < jz_end: R_max % 4 == 0
    }
    __syncthreads();
    bf16x8 dsf[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const uint2 lo = dsx[xi][2 * h2][lane], hi = dsx[xi][2 * h2 + 1][lane];
      dsf[h2] = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
    }
    prio_mfma();
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)       // independent accumulators per k-step
#pragma unroll
      for (int dt = 0; dt < 5; ++dt)
        if (dt < n_dt) acc[dt] = mfma32x32x16(lat_trans(cur, h2, 32 * (dt_lo + dt)), dsf[h2], acc[dt]);
    prio_valu();
  };
  for (int t = 0; t < n_tiles; ++t) {   // one loop body, the two buffers alternating
    char* const cur = (t & 1) ? kv1 : kv0;
    char* const nxt = (t & 1) ? kv0 : kv1;
    tile_step(cur, nxt, t);
  }

  float* dst = dq + hr * kLatD;
#pragma unroll
  for (int dt = 0; dt < 5; ++dt) {
    if (dt < n_dt) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d0 = 32 * (dt_lo + dt) + 8 * i4 + 4 * hl;
        float4 v = make_float4(acc[dt][4 * i4] * g.tau, acc[dt][4 * i4 + 1] * g.tau,
                               acc[dt][4 * i4 + 2] * g.tau, acc[dt][4 * i4 + 3] * g.tau);
        if (accumulate) {
          const float4 y = *reinterpret_cast<const float4*>(dst + d0);
          v.x += y.x;
          v.y += y.y;
          v.z += y.z;
          v.w += y.w;
        }
        *reinterpret_cast<float4*>(dst + d0) = v;
      }
    }
  }
}

// Rows of chunk c that the key tile starting at j0 sums over: [max(row_lo, c*cr, j0),
// min(row_hi, (c+1)*cr, r_len)).  Rows below j0 are skipped (their P / dS are zero for
// every key of the tile); the same rule decides, in xty_reduce, which partials exist.
__device__ __forceinline__ void xty_rows(int c, int cr, int row_lo, int row_hi, int j0, int rl, int& i_lo,
                                         int& i_hi) {
  i_lo = max(max(row_lo, c * cr), j0);
  i_hi = min(min(row_hi, (c + 1) * cr), rl);
}

// part[c][k][j][d] = sum over rows i of chunk c (xty_rows) and heads h of
// X[k][i][h][j] * Y[k][i][h][d].  Workgroup tile: 128 keys j x 128 dims d, four waves of
// 64 keys x 64 dims (each X^T and Y fragment feeds two MFMAs); inner dimension m = (i, h)
// in stages of 64 (16 MFMAs per wave), loaded straight into a ring of three LDS buffers
// (96 KiB) two stages ahead (the loads are issued from inline assembly and ordered by
// explicit vmcnt waits, one barrier per stage).  The Y tile is two 64-dim halves; past n_d the second half re-reads the first
// (its waves skip their MFMAs and writes), so every stage issues the same loads.
// Workgroups whose chunk has no rows for their key tile return at once and write nothing.
constexpr int kXtyM = 64;   // m rows per stage (a multiple of 32)
__global__ __launch_bounds__(256, 2) void xty_gemm(const uint16_t* __restrict__ X,
                                                   const uint16_t* __restrict__ Y, int ldY, int n_d,
                                                   float* __restrict__ part, int R, int K, int row_lo,
                                                   int row_hi, int j_hi, int cr, Geom g) {
  __shared__ __attribute__((aligned(1024))) char xb0[kXtyM * 128 * 2];
  __shared__ __attribute__((aligned(1024))) char xb1[kXtyM * 128 * 2];
  __shared__ __attribute__((aligned(1024))) char xb2[kXtyM * 128 * 2];
  __shared__ __attribute__((aligned(1024))) char yb0[2 * kXtyM * 64 * 2];
  __shared__ __attribute__((aligned(1024))) char yb1[2 * kXtyM * 64 * 2];
  __shared__ __attribute__((aligned(1024))) char yb2[2 * kXtyM * 64 * 2];
  constexpr int YH = kXtyM * 64 * 2;   // bytes of one 64-dim half tile
  const int n_jt = (j_hi + 127) / 128, n_dt = (n_d + 127) / 128;
  int64_t idx = blockIdx.x;
  const int dt = (int)(idx % n_dt);
  idx /= n_dt;
  const int jt = (int)(idx % n_jt);
  idx /= n_jt;
  const int k = (int)(idx % K);
  const int c = (int)(idx / K);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hl = lane >> 5, col = lane & 31;
  const int wk = wave & 1, wd = wave >> 1;   // this wave's 64 keys and 64 dims of the tile
  const int j0 = jt * 128, d0 = dt * 128;
  const bool second = d0 + 64 < n_d;         // the tile's second 64-dim half exists
  const bool live = wd == 0 || second;
  const int rl = g.r_len[k];
  int i_lo, i_hi;
  xty_rows(c, cr, row_lo, row_hi, j0, rl, i_lo, i_hi);
  if (i_hi <= i_lo) return;
  const int64_t m_lo = (int64_t)i_lo * kLatH, m_hi = (int64_t)i_hi * kLatH;
  const int n_steps = (int)((m_hi - m_lo) / kXtyM);   // kLatH is a multiple of kXtyM
  const char* xs = reinterpret_cast<const char*>(X + ((int64_t)k * R * kLatH + m_lo) * R + j0);
  const char* ys = reinterpret_cast<const char*>(Y + ((int64_t)k * R * kLatH + m_lo) * ldY + d0);
  const char* ys2 = second ? ys + 64 * 2 : ys;
  const uint32_t xstride = (uint32_t)R * 2, ystride = (uint32_t)ldY * 2;
  DirectLoadRows<128, kXtyM, 4> dlx;
  DirectLoadRows<64, kXtyM, 4> dly;
  dlx.init();
  dly.init();
  constexpr int LOADS = DirectLoadRows<128, kXtyM, 4>::PER_WAVE + 2 * DirectLoadRows<64, kXtyM, 4>::PER_WAVE;
  uint32_t xoff[2][2];                       // X^T fragments: key columns 64 wk + 32 kk .. +32
  Frag<128>::trans_offsets(64 * wk, xoff[0]);
  Frag<128>::trans_offsets(64 * wk + 32, xoff[1]);
  Frag<64> fy;
  fy.init();
  f32x16 acc[2][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[kk][n][e] = 0.0f;
  auto issue = [&](char* xb, char* yb, int st) {
    dlx.issue(lds_addr(xb), xs + (int64_t)st * kXtyM * xstride, kXtyM, xstride);
    dly.issue(lds_addr(yb), ys + (int64_t)st * kXtyM * ystride, kXtyM, ystride);
    dly.issue(lds_addr(yb + YH), ys2 + (int64_t)st * kXtyM * ystride, kXtyM, ystride);
  };
  // Stage st: its loads are done (only stage st+1's may be in flight), every wave is past
  // its reads of stage st-1's buffer, which then receives stage st+2.
  auto stage = [&](const char* xc, const char* yc, char* xn, char* yn, int st) {
    if (st + 1 < n_steps) wait_vmcnt_n<LOADS>(); else wait_vmcnt0();
    __syncthreads();
    if (st + 2 < n_steps) issue(xn, yn, st + 2);
    if (live) {
      const char* yh = yc + wd * YH;
      prio_mfma();
#pragma unroll
      for (int sub = 0; sub < kXtyM / 32; ++sub)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const bf16x8 a0 = Frag<128>::trans_at(xc, xoff[0], sub, h2);
          const bf16x8 a1 = Frag<128>::trans_at(xc, xoff[1], sub, h2);
#pragma unroll
          for (int n = 0; n < 2; ++n) {
            const bf16x8 b = fy.trans_frag(yh, sub, h2, n);
            acc[0][n] = mfma32x32x16(a0, b, acc[0][n]);
            acc[1][n] = mfma32x32x16(a1, b, acc[1][n]);
          }
        }
      prio_valu();
    }
  };
  issue(xb0, yb0, 0);
  if (n_steps > 1) issue(xb1, yb1, 1);
  for (int st = 0; st < n_steps; st += 3) {
    stage(xb0, yb0, xb2, yb2, st);
    if (st + 1 < n_steps) stage(xb1, yb1, xb0, yb0, st + 1);
    if (st + 2 < n_steps) stage(xb2, yb2, xb1, yb1, st + 2);
  }
  if (!live) return;
  // C layout: lane = dim column, registers = key rows
  float* pc = part + ((int64_t)c * K + k) * R * n_d;
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int d = d0 + 64 * wd + 32 * n + col;
    if (d >= n_d) continue;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int j = j0 + 64 * wk + 32 * kk + (e >> 2) * 8 + 4 * hl + (e & 3);
        if (j >= j_hi || j >= rl) continue;
        pc[(int64_t)j * n_d + d] = acc[kk][n][e];
      }
  }
}

// C[k][j][d] += alpha * sum over chunks c (in order) of part[c][k][j][d], for the chunks
// that had rows for j's key tile; j < min(j_hi, r_len[k]).  One thread per 4 dims.
__global__ __launch_bounds__(256) void xty_reduce(const float* __restrict__ part, float* __restrict__ C,
                                                  int ldC, int n_d, int R, int K, int row_lo, int row_hi,
                                                  int j_hi, int cr, int n_chunks, float alpha, Geom g) {
  const int n_d4 = n_d / 4;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_k = (int64_t)j_hi * n_d4;
  if (t >= per_k * K) return;
  const int k = (int)(t / per_k);
  const int64_t r = t % per_k;
  const int j = (int)(r / n_d4), d = 4 * (int)(r % n_d4);
  const int rl = g.r_len[k];
  if (j >= rl) return;
  const int j0 = j / 128 * 128;
  float4 sum = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int c = 0; c < n_chunks; ++c) {
    int i_lo, i_hi;
    xty_rows(c, cr, row_lo, row_hi, j0, rl, i_lo, i_hi);
    if (i_hi <= i_lo) continue;
    const float4 v = *reinterpret_cast<const float4*>(part + (((int64_t)c * K + k) * R + j) * n_d + d);
    sum.x += v.x;
    sum.y += v.y;
    sum.z += v.z;
    sum.w += v.w;
  }
  float4* dst = reinterpret_cast<float4*>(C + ((int64_t)k * R + j) * ldC + d);
  float4 y = *dst;
  y.x += alpha * sum.x;
  y.y += alpha * sum.y;
  y.z += alpha * sum.z;
  y.w += alpha * sum.w;
  *dst = y;
}

hipError_t launch_sparse_fwd(const Geom& g, int topk, const void* q, const void* latent_p,
                             const void* latent_r, const int32_t* sel, float* o, float* lse,
                             hipStream_t s) {
  hipLaunchKernelGGL(sparse_fwd<2>, dim3((unsigned)(g.K * g.R)), dim3(512), 0, s, g, topk,
                     (const uint16_t*)q, (const uint16_t*)latent_p, (const uint16_t*)latent_r, sel,
                     o, lse);
  return hipGetLastError();
}

hipError_t launch_sparse_dq(const Geom& g, int topk, const void* q, const void* latent_p,
                            const void* latent_r, const int32_t* sel, const void* d_o,
                            const float* lse, const float* Dvec, float* dq, uint16_t* p_r,
                            uint16_t* ds_r, int accumulate, hipStream_t s) {
  // both head tiles per workgroup (8 waves, two per SIMD): each gathered tile serves all
  // 64 heads
  hipLaunchKernelGGL(sparse_dq<2>, dim3((unsigned)(g.K * g.R)), dim3(512), 0, s, g, topk,
                     (const uint16_t*)q, (const uint16_t*)latent_p, (const uint16_t*)latent_r, sel,
                     (const uint16_t*)d_o, lse, Dvec, dq, p_r, ds_r, accumulate);
  return hipGetLastError();
}

hipError_t launch_xty(const uint16_t* X, const uint16_t* Y, int ldY, int n_d, float* C, int ldC,
                      float* part, const Geom& g, int row_lo, int row_hi, int j_hi, float alpha,
                      hipStream_t s) {
  if (j_hi <= 0) return hipSuccess;
  const int cr = xty_chunk_rows(g.R), n_chunks = xty_n_chunks(g.R);
  const int n_jt = (j_hi + 127) / 128, n_dt = (n_d + 127) / 128;
  hipLaunchKernelGGL(xty_gemm, dim3((unsigned)((int64_t)n_chunks * g.K * n_jt * n_dt)), dim3(256), 0, s, X, Y,
                     ldY, n_d, part, g.R, g.K, row_lo, row_hi, j_hi, cr, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)g.K * j_hi * (n_d / 4);
  hipLaunchKernelGGL(xty_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, C, ldC, n_d, g.R,
                     g.K, row_lo, row_hi, j_hi, cr, n_chunks, alpha, g);
  return hipGetLastError();
}

}  // namespace rr
