// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

#include "rr_internal.h"

namespace rr {

struct AttnPtrs {
  const void* q;      // [K][R][Hq][d_qk]
  const void* k_p;    // [P][Hkv][d_qk]
  const void* v_p;    // [P][Hkv][d_v]
  const void* k_r;    // [K][R][Hkv][d_qk]
  const void* v_r;    // [K][R][Hkv][d_v]
  const void* d_o;    // [K][R][Hq][d_v]           (backward)
  const float* lse;   // [K][R][Hq]                (backward; global statistics)
  const float* Dvec;  // [K][R][Hq]                (backward)
  float* part_o;      // [n_parts][K][R][Hq][d_v]  (forward partials)
  float* part_lse;    // [n_parts][K][R][Hq]
  float* dq_part;     // [n_parts][K][R][Hq][d_qk] (backward partials)
  float* dk_r;        // [K][R][Hkv][d_qk]
  float* dv_r;        // [K][R][Hkv][d_v]
};

// Forward partials: one softmax-statistics partial per prompt chunk plus the causal
// response part, for query rows [g.row_lo, g.row_hi).
hipError_t launch_fwd_partials(const Geom& g, int dtype, const AttnPtrs& a, hipStream_t s);

// Exact merge of n partials.  With `geom` non-null the rows are (k, r, h) of that
// geometry and padding rows (r >= r_len[k]) get O = 0, lse = -inf without reading parts.
hipError_t launch_merge(int n_parts, int64_t rows, int d_v, const float* part_o,
                        const float* part_lse, float* o, float* lse, const Geom* geom,
                        hipStream_t s);

// D = rowsum(dO * O) for rows [g.row_lo, g.row_hi); padding rows get 0.
hipError_t launch_bwd_pre(const Geom& g, int dtype, const float* o, const void* d_o,
                          float* Dvec, hipStream_t s);

// dQ partials over every part for query rows [g.row_lo, g.row_hi).
hipError_t launch_dq_partials(const Geom& g, int dtype, const AttnPtrs& a, hipStream_t s);

// dq (= or +=) sum over parts in part order, rows [g.row_lo, g.row_hi); padding rows 0.
hipError_t launch_dq_reduce(const Geom& g, const float* dq_part, float* dq, int accumulate,
                            hipStream_t s);

// dk_r/dv_r += contributions of query rows [g.row_lo, g.row_hi) to response keys
// [0, key_hi).
hipError_t launch_dkdv(const Geom& g, int dtype, const AttnPtrs& a, int key_hi, hipStream_t s);

// Zero rows [lo, hi) of every response in a [K][R][row_elems] fp32 tensor.
hipError_t launch_zero_rows(float* x, int K, int R, int lo, int hi, int64_t row_elems,
                            hipStream_t s);

// Latent-page sparse variant (k_topk.hip, k_sparse.hip).
// Exact top-k of every row by fp32 index scores (k_topk.hip); ws: the forward workspace of
// the latent problem (topk_ws layout).
hipError_t launch_topk(const float* q_idx, const float* k_idx, void* ws, int64_t P, int k, const Geom& g,
                       int32_t* idx_out, hipStream_t s);
hipError_t launch_sparse_fwd(const Geom& g, int topk, const void* q, const void* latent_p,
                             const void* latent_r, const int32_t* sel, float* o, float* lse,
                             hipStream_t s);
hipError_t launch_sparse_dq(const Geom& g, int topk, const void* q, const void* latent_p,
                            const void* latent_r, const int32_t* sel, const void* d_o,
                            const float* lse, const float* Dvec, float* dq, uint16_t* p_r,
                            uint16_t* ds_r, int accumulate, hipStream_t s);
// C[k][j][d] += alpha * sum over rows i in [max(row_lo, tile start), row_hi) and heads h of
// X[k][i][h][j] * Y[k][i][h][d] for j < min(j_hi, r_len[k]); `part` is the workspace of
// chunk partials ([xty_n_chunks][K][R][n_d] fp32), summed into C in chunk order.
hipError_t launch_xty(const uint16_t* X, const uint16_t* Y, int ldY, int n_d, float* C, int ldC,
                      float* part, const Geom& g, int row_lo, int row_hi, int j_hi, float alpha,
                      hipStream_t s);

// Full-sequence differential mode (k_kv_grads.hip): pack the rows of each KV head into
// the prompt-gradient stream (qs, os: [Hkv][n_rows][d]; sts: per 64-row stage lse*log2(e)
// then -D), then dk_p, dv_p of resident keys [key_lo, key_hi) (= or +=) over every stream
// row.
hipError_t launch_pg_pack(const Geom& g, const PgGeom& pg, int dtype, const void* q, const float* o,
                          const float* lse, const void* d_o, void* qs, void* os, float* sts, hipStream_t s);
// dk_r, dv_r += the causal response-key gradients of every row of every response (bf16),
// over the same packed stream.
// `slots`: kDkdvSlots partial slots of [128][d_qk + d_v] fp32 (free workspace).
hipError_t launch_resp_dkdv(const Geom& g, const PgGeom& pg, const void* k_r, const void* v_r, const void* qs,
                            const void* os, const float* sts, float* slots, float* dk_r, float* dv_r,
                            hipStream_t s);
hipError_t launch_prompt_dkdv(const Geom& g, const PgGeom& pg, int dtype, const void* k_p, const void* v_p,
                              const void* qs, const void* os, const float* sts, int64_t key_lo, int64_t key_hi,
                              float* dk_p, float* dv_p, int accumulate, hipStream_t s);

// LastKV previous-chunk blending (k_lastkv.hip): x_out = (1 - alpha_g) x_layer + alpha_g x_last
// over [rows][Hkv][d]; and its backward (d_layer, d_last optional; d_alpha [Hkv]).
hipError_t launch_lastkv_blend(int64_t rows, int Hkv, int d, int dtype, const float* alpha, const void* x_layer,
                               const void* x_last, void* x_out, hipStream_t s);
hipError_t launch_lastkv_blend_bwd(int64_t rows, int Hkv, int d, int dtype, const float* alpha,
                                   const void* x_layer, const void* x_last, const float* d_out, float* d_layer,
                                   float* d_last, float* d_alpha, int accumulate, hipStream_t s);

// acc[e] += scale * g[e], e < n.
hipError_t launch_axpy(float* acc, const float* g, int64_t n, float scale, hipStream_t s);

}  // namespace rr
