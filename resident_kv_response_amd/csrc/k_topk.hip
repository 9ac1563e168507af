// Sparse selection of the latent-page variant (gfx950): fp32 index scores and an exact
// per-query top-k.
//
// Source: ai.thesatyajit.com/articles/longstraw-2m-rl, section "Two incompatible
// architectures, same transaction": DSA index-key pages are kept resident and the sparse
// selection is rebuilt before attention.  Each query row i scores every prompt position
// j by sigma_ij = q_idx_i . k_idx_j (fp32) and keeps the top k positions; equal scores
// are ordered by position (lower first).
//
// index_scores_f32: sigma = q_idx k_idx^T on fp32 MFMA (v_mfma_f32_32x32x2_f32), written
// to the caller's workspace with row stride ld.  A wave owns 32 query rows (their q_idx
// fragments stay in registers) and streams 32-key tiles of k_idx straight from global
// memory; lanes 0-31 contract index dims 0..63 and lanes 32-63 dims 64..127, so each
// lane's operand is one contiguous 256-byte half row; the next tile's keys load while the
// current tile's 64 MFMAs run.
//
// topk_select: one workgroup per query row; scores are mapped to order-preserving
// unsigned keys.  Fast path (large rows): the key of a fixed descending rank in a sample
// of 64 evenly spread runs of 128 scores is a threshold that keeps about 3k positions;
// one pass over the row appends every position at or above it to a candidate list (one
// LDS atomic per wave and store), a radix select over the candidates finds the k-th
// largest key T and how many keys equal to T are taken, and the chosen positions are
// sorted in LDS.  The threshold only decides how much work the row takes, never which
// positions are chosen: a row whose candidate count falls outside [k, cap] (or with too
// many keys equal to T) runs the exact full-row path, radix passes over the whole row
// followed by a pass over contiguous per-thread ranges that writes positions in order.
#include "k_common.h"
#include "kernels.h"

namespace rr {

constexpr int kIdxDim = 128;
constexpr int kTopkThreads = 512, kTopkWaves = kTopkThreads / 64;
constexpr int kEqMax = kTopkSample - kTopkSortMax;   // positions tied at T kept for sorting

__global__ __launch_bounds__(256) void index_scores_f32(const float* __restrict__ q_idx,
                                                        const float* __restrict__ k_idx,
                                                        float* __restrict__ sigma, int64_t ld,
                                                        int rows, int64_t P, int key_tiles_per_wg) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int n_row_tiles = (rows + 127) / 128;
  const int rt = blockIdx.x % n_row_tiles;
  const int64_t kt0 = (int64_t)(blockIdx.x / n_row_tiles) * key_tiles_per_wg;
  const int64_t n_kt = (P + 31) / 32;
  const int row0 = rt * 128 + wave * 32;
  if (row0 >= rows) return;

  // A fragments: q_idx[row0 + col][64h + s], s = 0..63
  float qa[64];
  {
    const int r = min(row0 + col, rows - 1);
    const float4* src = reinterpret_cast<const float4*>(q_idx + (int64_t)r * kIdxDim + 64 * h);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float4 x = src[v];
      qa[4 * v + 0] = x.x;
      qa[4 * v + 1] = x.y;
      qa[4 * v + 2] = x.z;
      qa[4 * v + 3] = x.w;
    }
  }
  const int64_t kt_end = min(n_kt, kt0 + key_tiles_per_wg);
  const bool full_rows = row0 + 32 <= rows;
  // B fragments of key tile kt: k_idx[kt*32 + col][64h + s], s = 0..63 (a 256-byte half
  // row per lane); keys past P are redirected to P - 1 and not stored
  auto load_keys = [&](int64_t kt, float (&kb)[64]) {
    const int64_t key = kt * 32 + col;
    const int64_t kk = key < P ? key : P - 1;
    const float4* src = reinterpret_cast<const float4*>(k_idx + kk * kIdxDim + 64 * h);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float4 x = src[v];
      kb[4 * v + 0] = x.x;
      kb[4 * v + 1] = x.y;
      kb[4 * v + 2] = x.z;
      kb[4 * v + 3] = x.w;
    }
  };
  // scores of tile kt from kb while the next tile's keys load into kn
  auto tile = [&](int64_t kt, const float (&kb)[64], float (&kn)[64]) {
    if (kt + 1 < kt_end) load_keys(kt + 1, kn);
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int s = 0; s < 64; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[s], kb[s], acc, 0, 0, 0);
    const int64_t key = kt * 32 + col;
    if (key < P) {
      float* dst = sigma + (int64_t)row0 * ld + key;
      if (full_rows) {
#pragma unroll
        for (int i = 0; i < 16; ++i) dst[(int64_t)((i >> 2) * 8 + 4 * h + (i & 3)) * ld] = acc[i];
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = (i >> 2) * 8 + 4 * h + (i & 3);
          if (row0 + r < rows) dst[(int64_t)r * ld] = acc[i];
        }
      }
    }
  };
  float ka[64], kb2[64];
  if (kt0 < kt_end) load_keys(kt0, ka);
  for (int64_t kt = kt0; kt < kt_end; kt += 2) {
    tile(kt, ka, kb2);
    if (kt + 1 < kt_end) tile(kt + 1, kb2, ka);
  }
}

// Order-preserving map of an fp32 score to an unsigned key (larger score -> larger key);
// +0 and -0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t b = __float_as_uint(f);
  if ((b & 0x7FFFFFFFu) == 0) return 0x80000000u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Exclusive scan over the workgroup's threads (in thread order); returns the exclusive
// prefix and writes the total to *total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < kTopkWaves; ++w) {
    base += w < wave ? scratch[w] : 0;
    tot += scratch[w];
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

struct TopkShared {
  int hist[2048];
  int scan[kTopkWaves];
  int sel_bin, sel_above;
  int n_cand, n_gt, n_eq;
  uint32_t cmax;
};

// The `rank`-th largest (1-based) of n keys whose values lie below 2^nbits, by radix
// passes of up to 11 bits from the top: returns it in T and, in need, how many keys equal
// to T belong to the top `rank`.  Requires 1 <= rank <= n.  Every thread of the
// workgroup calls it; key_at(i) may read global or shared memory.
template <class F>
__device__ void radix_kth(F key_at, int64_t n, int rank, int nbits, TopkShared& sh, uint32_t& T,
                          int& need_out) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0;
  int need = rank, hi = nbits;
  while (hi > 0) {
    const int w = hi < 11 ? hi : 11, shift = hi - w, nb = 1 << w;
    for (int b = tid; b < nb; b += kTopkThreads) sh.hist[b] = 0;
    __syncthreads();
    for (int64_t i = tid; i < n; i += kTopkThreads) {
      const uint32_t u = key_at(i);
      if (hi == 32 || (u >> hi) == prefix) atomicAdd(&sh.hist[(u >> shift) & (nb - 1)], 1);
    }
    __syncthreads();
    // bins from the top: thread t owns bins nb-1-t*per .. nb-per-t*per
    const int per = (nb + kTopkThreads - 1) / kTopkThreads;
    int s = 0;
    for (int q = 0; q < per; ++q) {
      const int b = nb - 1 - (tid * per + q);
      s += b >= 0 ? sh.hist[b] : 0;
    }
    int tot;
    const int base = block_exclusive_scan(s, sh.scan, &tot);
    if (base < need && need <= base + s) {
      int c = base;
      for (int q = 0; q < per; ++q) {
        const int b = nb - 1 - (tid * per + q);
        if (c + sh.hist[b] >= need) {
          sh.sel_bin = b;
          sh.sel_above = c;
          break;
        }
        c += sh.hist[b];
      }
    }
    __syncthreads();
    prefix = (prefix << w) | (uint32_t)sh.sel_bin;
    need -= sh.sel_above;
    hi = shift;
    __syncthreads();
  }
  T = prefix;
  need_out = need;
}

// Ascending bitonic sort of n (a power of two) ints in shared memory.
__device__ void bitonic_sort(int* a, int n) {
  for (int size = 2; size <= n; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < n / 2; t += kTopkThreads) {
        const int i = 2 * t - (t & (stride - 1)), j = i + stride;
        const bool up = (i & size) == 0;
        const int x = a[i], y = a[j];
        if ((x > y) == up) {
          a[i] = y;
          a[j] = x;
        }
      }
      __syncthreads();
    }
}

__device__ __forceinline__ int pow2_ceil(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// Exact selection over the whole row: radix passes, then a pass over contiguous
// per-thread ranges (a block-wide scan gives each thread its output offset) that writes
// the chosen positions in ascending order.
__device__ void full_row_select(const float* srow, int64_t P, int k, int32_t* out, TopkShared& sh) {
  const int tid = threadIdx.x;
  uint32_t T;
  int need;
  radix_kth([&](int64_t j) { return order_key(srow[j]); }, P, k, 32, sh, T, need);
  const int64_t chunk = (P + kTopkThreads - 1) / kTopkThreads;
  const int64_t j0 = min(P, chunk * tid), j1 = min(P, j0 + chunk);
  int n_gt = 0, n_eq = 0;
  for (int64_t j = j0; j < j1; ++j) {
    const uint32_t u = order_key(srow[j]);
    n_gt += u > T;
    n_eq += u == T;
  }
  int tot;
  const int eq_base = block_exclusive_scan(n_eq, sh.scan, &tot);
  const int eq_take = max(0, min(n_eq, need - eq_base));
  const int out_base = block_exclusive_scan(n_gt + eq_take, sh.scan, &tot);
  int pos = out_base, eq_seen = 0;
  for (int64_t j = j0; j < j1 && pos < out_base + n_gt + eq_take && pos < k; ++j) {
    const uint32_t u = order_key(srow[j]);
    if (u > T) {
      out[pos++] = (int32_t)j;
    } else if (u == T) {
      if (eq_seen < eq_take) out[pos++] = (int32_t)j;
      ++eq_seen;
    }
  }
}

// Wave-aggregated append: lanes with pred set get consecutive slots from *counter.
__device__ __forceinline__ int wave_append_slot(bool pred, int* counter) {
  const int lane = threadIdx.x & 63;
  const uint64_t m = __ballot(pred);
  int base = 0;
  if (lane == 0) base = atomicAdd(counter, __popcll(m));
  base = __shfl(base, 0, 64);
  return base + __popcll(m & ((1ull << lane) - 1));
}

__global__ __launch_bounds__(kTopkThreads) void topk_select(const float* __restrict__ sigma, int64_t ld,
                                                            int64_t P, int k, Geom g,
                                                            int32_t* __restrict__ idx_out,
                                                            uint32_t* __restrict__ cand_key,
                                                            int32_t* __restrict__ cand_pos, int fast,
                                                            int sample_rank, int cap) {
  __shared__ TopkShared sh;
  __shared__ uint32_t buf[kTopkSample];    // sample keys; later sorted positions | tied positions
  const int row = blockIdx.x;              // (k, r) flattened
  if (row >= g.K * g.R) return;
  const int kk = row / g.R, r = row % g.R;
  int32_t* out = idx_out + (int64_t)row * k;
  if (r < g.row_lo || r >= g.row_hi) return;
  const int tid = threadIdx.x, lane = tid & 63;
  if (r >= g.r_len[kk]) {                // padding row
    for (int t = tid; t < k; t += kTopkThreads) out[t] = -1;
    return;
  }
  const float* srow = sigma + (int64_t)row * ld;
  if (!fast) {
    full_row_select(srow, P, k, out, sh);
    return;
  }

  // 1. threshold from the sample: 64 runs of 128 scores, run q starting near q (P-128)/63
  {
    const int run = tid >> 3, off = (tid & 7) * 16;
    const int64_t start = ((int64_t)run * (P - 128) / 63) & ~(int64_t)3;
    const float4* src = reinterpret_cast<const float4*>(srow + start + off);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float4 x = src[v];
      buf[16 * tid + 4 * v + 0] = order_key(x.x);
      buf[16 * tid + 4 * v + 1] = order_key(x.y);
      buf[16 * tid + 4 * v + 2] = order_key(x.z);
      buf[16 * tid + 4 * v + 3] = order_key(x.w);
    }
  }
  if (tid == 0) {
    sh.n_cand = 0;
    sh.n_gt = 0;
    sh.n_eq = 0;
    sh.cmax = 0;
  }
  __syncthreads();
  uint32_t t_lo;
  {
    int unused;
    radix_kth([&](int64_t i) { return buf[i]; }, kTopkSample, sample_rank, 32, sh, t_lo, unused);
  }

  // 2. candidates: every position whose key is >= t_lo (slots past cap are counted only)
  uint32_t* ck = cand_key + (int64_t)row * cap;
  int32_t* cp = cand_pos + (int64_t)row * cap;
  uint32_t lmax = 0;
  auto consider = [&](bool valid, float x, int64_t j) {
    const uint32_t u = order_key(x);
    const bool pred = valid && u >= t_lo;
    if (__ballot(pred)) {
      const int slot = wave_append_slot(pred, &sh.n_cand);
      if (pred) {
        if (slot < cap) {
          ck[slot] = u - t_lo;
          cp[slot] = (int32_t)j;
        }
        lmax = max(lmax, u - t_lo);
      }
    }
  };
  const float4* s4 = reinterpret_cast<const float4*>(srow);
  const int64_t n4 = P >> 2;
  constexpr int U = 4;
  // trip counts are uniform across the workgroup so every lane reaches each ballot
  for (int64_t b0 = 0; b0 < n4; b0 += (int64_t)U * kTopkThreads) {
    float4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i4 = b0 + (int64_t)u * kTopkThreads + tid;
      x[u] = s4[i4 < n4 ? i4 : n4 - 1];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i4 = b0 + (int64_t)u * kTopkThreads + tid;
      const bool v = i4 < n4;
      consider(v, x[u].x, 4 * i4 + 0);
      consider(v, x[u].y, 4 * i4 + 1);
      consider(v, x[u].z, 4 * i4 + 2);
      consider(v, x[u].w, 4 * i4 + 3);
    }
  }
  for (int64_t j0 = 4 * n4; j0 < P; j0 += kTopkThreads) {   // tail of P % 4 positions
    const int64_t j = j0 + tid;
    consider(j < P, j < P ? srow[j] : 0.0f, j);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) lmax = max(lmax, (uint32_t)__shfl_xor((int)lmax, off, 64));
  if (lane == 0) atomicMax(&sh.cmax, lmax);
  __syncthreads();
  const int n_c = sh.n_cand;
  if (n_c < k || n_c > cap) {            // the sample misled this row: exact full-row path
    full_row_select(srow, P, k, out, sh);
    return;
  }

  // 3. exact k-th largest among the candidates (keys relative to t_lo)
  uint32_t T;
  int need;
  const int nbits = sh.cmax ? 32 - __clz(sh.cmax) : 0;
  radix_kth([&](int64_t i) { return ck[i]; }, n_c, k, nbits, sh, T, need);

  // 4. positions above T, and the positions tied at T (the lowest `need` of them are taken)
  int* sorted = reinterpret_cast<int*>(buf);                 // [kTopkSortMax]
  int* tied = reinterpret_cast<int*>(buf) + kTopkSortMax;    // [kEqMax]
  for (int64_t i0 = 0; i0 < n_c; i0 += kTopkThreads) {
    const int64_t i = i0 + tid;
    const bool v = i < n_c;
    const uint32_t u = v ? ck[i] : 0;
    const int32_t j = v ? cp[i] : 0;
    const bool gt = v && u > T, eq = v && u == T;
    if (__ballot(gt)) {
      const int slot = wave_append_slot(gt, &sh.n_gt);
      if (gt && slot < kTopkSortMax) sorted[slot] = j;
    }
    if (__ballot(eq)) {
      const int slot = wave_append_slot(eq, &sh.n_eq);
      if (eq && slot < kEqMax) tied[slot] = j;
    }
  }
  __syncthreads();
  const int n_eq = sh.n_eq;
  if (n_eq > kEqMax) {                   // too many ties at T to sort here
    full_row_select(srow, P, k, out, sh);
    return;
  }
  if (n_eq > need) {
    const int n2 = pow2_ceil(n_eq);
    for (int t = n_eq + tid; t < n2; t += kTopkThreads) tied[t] = 0x7FFFFFFF;
    __syncthreads();
    bitonic_sort(tied, n2);
  }
  const int n_gt = k - need;             // == sh.n_gt
  for (int t = tid; t < need; t += kTopkThreads) sorted[n_gt + t] = tied[t];
  const int k2 = pow2_ceil(k);
  for (int t = k + tid; t < k2; t += kTopkThreads) sorted[t] = 0x7FFFFFFF;
  __syncthreads();
  bitonic_sort(sorted, k2);
  for (int t = tid; t < k; t += kTopkThreads) out[t] = sorted[t];
}

hipError_t launch_index_scores(const float* q_idx, const float* k_idx, float* sigma, int64_t ld,
                               int rows, int64_t P, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int n_row_tiles = (rows + 127) / 128;
  const int64_t n_kt = (P + 31) / 32;
  // about 2048 workgroups in total
  const int64_t splits = max((int64_t)1, min(n_kt, (int64_t)(2048 / n_row_tiles)));
  const int per = (int)((n_kt + splits - 1) / splits);
  const int64_t n_splits = (n_kt + per - 1) / per;
  hipLaunchKernelGGL(index_scores_f32, dim3((unsigned)(n_row_tiles * n_splits)), dim3(256), 0, s, q_idx,
                     k_idx, sigma, ld, rows, P, per);
  return hipGetLastError();
}

hipError_t launch_topk(void* ws, int64_t P, int k, const Geom& g, int32_t* idx_out, hipStream_t s) {
  const TopkPlan t = topk_plan(P, k);
  const size_t rows = (size_t)g.K * g.R;
  char* base = static_cast<char*>(ws);
  const float* sigma = reinterpret_cast<const float*>(base);
  const size_t o1 = align_up(rows * (size_t)t.ld * sizeof(float), 256);
  const size_t o2 = o1 + align_up(rows * (size_t)t.cap * sizeof(uint32_t), 256);
  uint32_t* ck = t.fast ? reinterpret_cast<uint32_t*>(base + o1) : nullptr;
  int32_t* cp = t.fast ? reinterpret_cast<int32_t*>(base + o2) : nullptr;
  hipLaunchKernelGGL(topk_select, dim3((unsigned)rows), dim3(kTopkThreads), 0, s, sigma, t.ld, P, k, g,
                     idx_out, ck, cp, t.fast, t.sample_rank, t.cap);
  return hipGetLastError();
}

}  // namespace rr
