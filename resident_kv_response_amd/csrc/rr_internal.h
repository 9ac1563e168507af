// Internal declarations shared by the host library sources (not part of the C ABI).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/rr_attn.h"

namespace rr {

// Geometry of one launch, passed to kernels by value.
struct Geom {
  int64_t P;          // resident prompt positions
  int64_t chunk;      // prompt chunk length
  int32_t R;          // row stride (R_max)
  int32_t K;          // responses in the microbatch
  int32_t Hq, Hkv, grp;
  int32_t dqk, dv;
  int32_t n_chunks;   // prompt chunks
  int32_t n_parts;    // n_chunks + 1 (the response's causal keys are the last part)
  int32_t row_lo;     // query rows [row_lo, row_hi) handled by this launch
  int32_t row_hi;
  float tau;          // softmax scale
  float c2;           // tau * log2(e): scores in base-2 units
  int32_t resp_keys;  // 1: the response's own causal keys form the last part; 0: another
                      // prompt shard owns them and the last part is empty
  int32_t r_len[RR_MAX_K];
  // Partial buffers (forward O_c / lse_c, dQ partials): the values of part c for row
  // m = (k R + r) Hq + h start at row index c * part_step + m * row_step (times the head
  // dim for O and dQ).  Part-major (part_step = K R Hq, row_step = 1) is the exported
  // layout; the workspace holds them row-major (part_step = 1, row_step = n_parts), so the
  // merge and the dQ reduction read each row's parts as one contiguous run.
  int64_t part_step;
  int64_t row_step;
};

inline void set_parts_row_major(Geom& g) {
  g.part_step = 1;
  g.row_step = g.n_parts;
}

// ---- validation (HIP-free; rr_validate.cpp) ----------------------------------------
int set_error(int code, const char* fmt, ...);
void clear_error();
int validate_problem(const rr_problem* p);
int64_t n_chunks_of(const rr_problem* p);
int32_t n_parts_of(const rr_problem* p);
size_t ws_fwd_bytes(const rr_problem* p, bool exported);
size_t ws_bwd_bytes(const rr_problem* p);
size_t ws_pds_bytes(const rr_problem* p);
int validate_fwd(const rr_problem* p, const rr_resident* kv, const void* q, const void* k_r,
                 const void* v_r, const int32_t* r_len, const float* q_idx, const float* o,
                 const float* lse, const float* part_o, const float* part_lse,
                 const int32_t* topk_idx, const void* ws, size_t ws_bytes);
int validate_bwd(const rr_problem* p, const rr_resident* kv, const void* q, const void* k_r,
                 const void* v_r, const int32_t* r_len, const int32_t* topk_idx,
                 const float* o, const float* lse, const void* d_o, const float* dq,
                 const float* dk_r, const float* dv_r, int32_t accumulate, int32_t block_idx,
                 const void* ws, size_t ws_bytes);
int validate_merge(int32_t n_parts, int64_t rows, int32_t d_v, const float* part_o,
                   const float* part_lse, const float* o, const float* lse);
int validate_accum(const rr_accum* acc, int32_t member_g, const rr_grad_tag* tag,
                   const float* const* grads, const int64_t* n_elems);
uint64_t tag_seal(const rr_grad_tag* t);
void write_tag(const rr_resident* kv, rr_grad_tag* t);

// Kinds of memory a pointer lookup can report (the HIP runtime's memory types, mapped in
// rr_api.cpp), and whether a kernel may dereference such a pointer.
enum class PtrKind { Unregistered, Host, Device, Managed, Array, Unified, Unknown };
bool ptr_accessible(bool query_ok, PtrKind kind, bool has_device_ptr);
Geom make_geom(const rr_problem* p, const int32_t* r_len);
int rr_attn_fwd_impl(const rr_problem* p, const rr_resident* kv, const void* q, const void* k_r,
                     const void* v_r, const int32_t* r_len, const float* q_idx, float* o, float* lse,
                     float* part_o, float* part_lse, int32_t* topk_idx, void* ws, size_t ws_bytes,
                     void* stream, bool ws_is_scratch);
int rr_attn_bwd_impl(const rr_problem* p, const rr_resident* kv, const void* q, const void* k_r,
                     const void* v_r, const int32_t* r_len, const int32_t* topk_idx, const float* o,
                     const float* lse, const void* d_o, float* dq, float* dk_r, float* dv_r,
                     int32_t accumulate, int32_t block_idx, void* ws, size_t ws_bytes, void* stream);

// Packed row stream of the key-parallel K/V-gradient kernels: the rows of each KV head,
// response after response.  Response k contributes its flattened rows m = r * grp + hh
// from m_lo (a multiple of 64, the stage holding row row_lo) up to min(r_len[k], row_hi) *
// grp, padded to a multiple of 64; rows outside [row_lo, min(r_len[k], row_hi)) are empty
// (they contribute nothing).  off[k] is response k's first stream row; off[K] = n_rows.
struct PgGeom {
  int32_t n_rows;
  int32_t m_lo;
  int32_t off[RR_MAX_K + 1];
};
PgGeom make_pg_geom(const rr_problem* p, const int32_t* r_len, int32_t row_lo, int32_t row_hi);
// The response dK/dV kernel cuts each 128-key tile's run of stream stages into segments of
// at most `seg` stages, one workgroup each, so that long and short tiles cost alike; the
// first segment of a tile adds its sum to dk_r / dv_r, every later one writes a partial
// slot ([128 keys][d] fp32 for dK, then for dV) that an ordered reduction adds afterwards.
// seg is chosen per response so that each response of a launch has at most
// kDkdvItemsTarget later segments, which the workspace's kDkdvSlots slots per response
// bound with room to spare.
constexpr int kDkdvItemsTarget = 768;
constexpr int kDkdvSlots = 1024;
constexpr int kDkdvMinSeg = 8;
// Slots a response of at most R_max rows can need: kDkdvSlots, or fewer when its
// stage-tiles (Hkv x 128-key tiles x 64-row stages) divided by kDkdvMinSeg are fewer.
inline int64_t dkdv_slots_per_response(int64_t R_max, int64_t Hkv, int64_t grp) {
  const int64_t stage_tiles = Hkv * ((R_max + 127) / 128) * ((R_max * grp + 63) / 64);
  const int64_t by_size = stage_tiles / kDkdvMinSeg;
  return by_size < kDkdvSlots ? by_size : kDkdvSlots;
}
size_t ws_dkdv_slots_bytes(const rr_problem* p);
int validate_blend(int64_t rows, int32_t Hkv, int32_t d, int32_t dtype, const float* alpha,
                   const void* x_layer, const void* x_last, const void* x_out);
int validate_blend_bwd(int64_t rows, int32_t Hkv, int32_t d, int32_t dtype, const float* alpha,
                       const void* x_layer, const void* x_last, const float* d_out, const float* d_layer,
                       const float* d_last, const float* d_alpha, int32_t accumulate);
size_t ws_prompt_bytes(const rr_problem* p);
int validate_prompt_grads(const rr_problem* p, const rr_resident* kv, const void* q,
                          const int32_t* r_len, const float* o, const float* lse, const void* d_o,
                          int64_t key_lo, int64_t key_hi, const float* dk_p, const float* dv_p,
                          int32_t accumulate, const void* ws, size_t ws_bytes);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Row chunks of the latent response-pair GEMM (dK_r, dV_r): the response rows are split
// into at most 16 chunks of at least 256 rows; each chunk's partial product is written to
// the workspace and the partials are summed in chunk order.
inline int xty_chunk_rows(int R_max) {
  const int n = (R_max + 255) / 256;
  const int n_chunks = n < 16 ? n : 16;
  return (R_max + n_chunks - 1) / n_chunks;
}
inline int xty_n_chunks(int R_max) {
  const int cr = xty_chunk_rows(R_max);
  return (R_max + cr - 1) / cr;
}

// Plan of the per-row top-k selection (k_topk.hip).  The fp32 index score of (row, position)
// is one fixed-order chain of 128 fused multiply-adds; the selection is the top k by it,
// equal scores ordered by position.  Fast path (P >= kScreenMinP): a sample of
// kTopkSample positions per row, scored by the screen, gives a threshold expected to keep
// about 3k positions; a screen over every position (products of the bf16 hi/lo parts,
// within a stated bound of the fp32 score) keeps those at or above it as candidates, key
// range by key range, at most `cap` per row; the selection is then made exactly among
// them, computing the fp32 score of every candidate the bound leaves undecided.  Rows the
// screen cannot decide, and every row below kScreenMinP, take the exact full-row path.
constexpr int kTopkSample = 8192;
constexpr int kTopkSortMax = 4096;
constexpr int64_t kScreenMinP = 65536;
constexpr int kScreenKeys = 32;          // keys per screen tile
constexpr int kScreenRows = 256;         // query rows per screen workgroup
struct TopkPlan {
  int fast;            // 1: sample + screen path for this (P, k)
  int sample_rank;     // descending rank in the sample that sets the threshold
  int cap;             // candidate slots per row
  int n_splits;        // key ranges of the screen, each a run of whole 32-key tiles
  int64_t tiles_per_split;
};
inline TopkPlan topk_plan(int64_t P, int k) {
  TopkPlan t{};
  const int64_t rs = (3 * (int64_t)k * kTopkSample + P - 1) / P;
  t.sample_rank = (int)(rs < 32 ? 32 : rs);
  t.fast = P >= kScreenMinP && k <= kTopkSortMax && t.sample_rank <= kTopkSample / 4;
  if (t.fast) {
    const int64_t expect = (int64_t)t.sample_rank * P / kTopkSample;   // candidates expected
    t.cap = (int)((2 * expect + 1024 + 255) / 256 * 256);
    const int64_t n_kt = (P + kScreenKeys - 1) / kScreenKeys;
    const int64_t want = 128;                                         // key ranges
    t.tiles_per_split = (n_kt + want - 1) / want;
    t.n_splits = (int)((n_kt + t.tiles_per_split - 1) / t.tiles_per_split);
  }
  return t;
}

// Forward workspace of the latent selection: per row the threshold and the candidate
// count, the key-norm maximum of each key range, then one region that first holds the
// sample scores [rows][kTopkSample] and then the candidates (keys [rows][cap], positions
// [rows][cap]).
struct TopkWs {
  size_t thr, cnt, knorm, region, total;
};
inline TopkWs topk_ws(int64_t P, int k, size_t rows) {
  const TopkPlan t = topk_plan(P, k);
  TopkWs w{};
  w.thr = 0;
  w.cnt = align_up(rows * 4, 256);
  w.knorm = w.cnt + align_up(rows * 4, 256);
  w.region = w.knorm + align_up((size_t)(t.fast ? t.n_splits : 1) * 4, 256);
  const size_t samp = t.fast ? rows * (size_t)kTopkSample * 4 : 0;
  const size_t cand = t.fast ? 2 * align_up(rows * (size_t)t.cap * 4, 256) : 0;
  w.total = w.region + align_up(samp > cand ? samp : cand, 256);
  return w;
}

}  // namespace rr
