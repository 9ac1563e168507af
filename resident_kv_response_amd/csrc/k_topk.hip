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
// to the caller's workspace.  A wave owns 32 query rows (their q_idx fragments stay in
// registers) and streams 32-key tiles of k_idx straight from global memory; lanes 0-31
// contract index dims 0..63 and lanes 32-63 dims 64..127, so each lane's operand is one
// contiguous 256-byte half row.
//
// topk_select: one workgroup per query row.  Scores are mapped to order-preserving
// unsigned keys; three radix passes (11, 11, 10 bits) over the row find the k-th largest
// key T and how many keys equal to T must be taken; a final pass over contiguous
// per-thread ranges (a block-wide scan gives each thread its output offset) writes the
// selected positions in ascending order.
#include "k_common.h"
#include "kernels.h"

namespace rr {

constexpr int kIdxDim = 128;

typedef float f32x4v __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void index_scores_f32(const float* __restrict__ q_idx,
                                                        const float* __restrict__ k_idx,
                                                        float* __restrict__ sigma, int rows,
                                                        int64_t P, int key_tiles_per_wg) {
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
  for (int64_t kt = kt0; kt < kt_end; ++kt) {
    const int64_t key = kt * 32 + col;
    const int64_t kk = key < P ? key : P - 1;
    const float4* src = reinterpret_cast<const float4*>(k_idx + kk * kIdxDim + 64 * h);
    float kb[64];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float4 x = src[v];
      kb[4 * v + 0] = x.x;
      kb[4 * v + 1] = x.y;
      kb[4 * v + 2] = x.z;
      kb[4 * v + 3] = x.w;
    }
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
#pragma unroll
    for (int s = 0; s < 64; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[s], kb[s], acc, 0, 0, 0);
    if (key < P) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = row0 + (i >> 2) * 8 + 4 * h + (i & 3);
        if (r < rows) sigma[(int64_t)r * P + key] = acc[i];
      }
    }
  }
}

// Order-preserving map of an fp32 score to an unsigned key (larger score -> larger key);
// +0 and -0 map to the same key.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t b = __float_as_uint(f);
  if ((b & 0x7FFFFFFFu) == 0) return 0x80000000u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Exclusive scan over the 256 threads of the block (in thread order); returns the
// exclusive prefix and writes the block total to *total.
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
  int base = 0;
  for (int w = 0; w < wave; ++w) base += scratch[w];
  const int tot = scratch[0] + scratch[1] + scratch[2] + scratch[3];
  __syncthreads();
  *total = tot;
  return base + x - v;
}

__global__ __launch_bounds__(256) void topk_select(const float* __restrict__ sigma, int64_t P,
                                                   int k, int R, int K, Geom g,
                                                   int32_t* __restrict__ idx_out) {
  __shared__ int hist[2048];
  __shared__ int scan_scratch[4];
  __shared__ int sel_bin, sel_above;
  const int row = blockIdx.x;            // (k, r) flattened
  if (row >= K * R) return;
  const int kk = row / R, r = row % R;
  int32_t* out = idx_out + (int64_t)row * k;
  if (r < g.row_lo || r >= g.row_hi) return;
  if (r >= g.r_len[kk]) {                // padding row
    for (int t = threadIdx.x; t < k; t += 256) out[t] = -1;
    return;
  }
  const float* srow = sigma + (int64_t)row * P;
  const int tid = threadIdx.x;

  uint32_t prefix = 0;
  int need = k;
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass], nb = 1 << widths[pass];
    for (int b = tid; b < nb; b += 256) hist[b] = 0;
    __syncthreads();
    const int hi_shift = shift + widths[pass];
    for (int64_t j = tid; j < P; j += 256) {
      const uint32_t u = order_key(srow[j]);
      const bool match = pass == 0 || (u >> hi_shift) == prefix;
      if (match) atomicAdd(&hist[(u >> shift) & (nb - 1)], 1);
    }
    __syncthreads();
    // bins from the top: thread t owns bins [nb - per*(t+1), nb - per*t)
    const int per = nb / 256;
    int s = 0;
    for (int q = 0; q < per; ++q) s += hist[nb - 1 - (tid * per + q)];
    int tot;
    const int base = block_exclusive_scan(s, scan_scratch, &tot);
    if (base < need && need <= base + s) {
      int c = base;
      for (int q = 0; q < per; ++q) {
        const int b = nb - 1 - (tid * per + q);
        if (c + hist[b] >= need) {
          sel_bin = b;
          sel_above = c;
          break;
        }
        c += hist[b];
      }
    }
    __syncthreads();
    prefix = (prefix << widths[pass]) | (uint32_t)sel_bin;
    need -= sel_above;
    __syncthreads();
  }
  const uint32_t T = prefix;   // the k-th largest key; `need` keys equal to T are taken

  // contiguous per-thread ranges keep the output in ascending position order
  const int64_t chunk = (P + 255) / 256;
  const int64_t j0 = min(P, chunk * tid), j1 = min(P, j0 + chunk);
  int n_gt = 0, n_eq = 0;
  for (int64_t j = j0; j < j1; ++j) {
    const uint32_t u = order_key(srow[j]);
    n_gt += u > T;
    n_eq += u == T;
  }
  int tot;
  const int eq_base = block_exclusive_scan(n_eq, scan_scratch, &tot);
  const int eq_take = max(0, min(n_eq, need - eq_base));
  const int out_base = block_exclusive_scan(n_gt + eq_take, scan_scratch, &tot);
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

hipError_t launch_index_scores(const float* q_idx, const float* k_idx, float* sigma, int rows,
                               int64_t P, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int n_row_tiles = (rows + 127) / 128;
  const int64_t n_kt = (P + 31) / 32;
  // about 2048 workgroups in total
  const int64_t splits = max((int64_t)1, min(n_kt, (int64_t)(2048 / n_row_tiles)));
  const int per = (int)((n_kt + splits - 1) / splits);
  const int64_t n_splits = (n_kt + per - 1) / per;
  hipLaunchKernelGGL(index_scores_f32, dim3((unsigned)(n_row_tiles * n_splits)), dim3(256), 0, s, q_idx,
                     k_idx, sigma, rows, P, per);
  return hipGetLastError();
}

hipError_t launch_topk(const float* sigma, int64_t P, int k, const Geom& g, int32_t* idx_out,
                       hipStream_t s) {
  hipLaunchKernelGGL(topk_select, dim3((unsigned)(g.K * g.R)), dim3(256), 0, s, sigma, P, k, g.R, g.K, g,
                     idx_out);
  return hipGetLastError();
}

}  // namespace rr
