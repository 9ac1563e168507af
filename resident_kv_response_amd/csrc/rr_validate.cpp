// Argument validation, workspace sizing and error reporting.  HIP-free: every check
// here runs on the host before anything is launched, so an invalid call has no side
// effects on the device.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "rr_internal.h"

namespace rr {

static thread_local char g_err[512] = "";

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = '\0'; }

const char* last_error() { return g_err; }

int validate_problem(const rr_problem* p) {
  if (!p) return set_error(RR_E_NULL, "problem is NULL");
  if (p->P < 0) return set_error(RR_E_SHAPE, "P must be >= 0 (got %lld)", (long long)p->P);
  if (p->R_max < 1) return set_error(RR_E_SHAPE, "R_max must be >= 1 (got %d)", p->R_max);
  if (p->K < 1 || p->K > RR_MAX_K)
    return set_error(RR_E_SHAPE, "K must be in [1, %d] (got %d)", RR_MAX_K, p->K);
  if (p->Hq < 1 || p->Hkv < 1)
    return set_error(RR_E_SHAPE, "Hq and Hkv must be >= 1 (got %d, %d)", p->Hq, p->Hkv);
  if (p->Hq % p->Hkv != 0)
    return set_error(RR_E_SHAPE, "Hq (%d) must be a multiple of Hkv (%d)", p->Hq, p->Hkv);
  if (p->chunk < 1) return set_error(RR_E_SHAPE, "chunk must be >= 1 (got %lld)", (long long)p->chunk);
  if (p->block < 1) return set_error(RR_E_SHAPE, "block must be >= 1 (got %d)", p->block);
  if (!(p->tau > 0.0f) || !std::isfinite(p->tau))
    return set_error(RR_E_SHAPE, "tau must be finite and > 0");
  if (p->dtype != RR_F32 && p->dtype != RR_BF16)
    return set_error(RR_E_SHAPE, "dtype must be RR_F32 or RR_BF16 (got %d)", p->dtype);
  if (p->topk < 0) return set_error(RR_E_SHAPE, "topk must be >= 0");
  if (p->flags & ~RR_FLAG_SHARD_NO_RESPONSE) return set_error(RR_E_SHAPE, "unknown flags 0x%x", p->flags);
  if (p->latent) {
    if (p->dtype != RR_BF16) return set_error(RR_E_UNSUPPORTED, "latent pages need bf16 inputs");
    if (p->d_qk != 576 || p->d_v != 512 || p->Hkv != 1 || p->Hq != 64)
      return set_error(RR_E_UNSUPPORTED, "latent pages are built for d_qk=576, d_v=512, Hkv=1, Hq=64 "
                       "(got %d, %d, %d, %d)", p->d_qk, p->d_v, p->Hkv, p->Hq);
    if (p->topk < 32 || p->topk % 32 != 0 || p->topk > p->P || p->topk > 4096)
      return set_error(RR_E_SHAPE, "latent top-k must be a multiple of 32 in [32, min(P, 4096)] (got %d)",
                       p->topk);
    if (p->idx_dim != 128) return set_error(RR_E_UNSUPPORTED, "index keys must be 128 wide (got %d)", p->idx_dim);
    if (p->R_max % 8 != 0) return set_error(RR_E_SHAPE, "latent pages need R_max %% 8 == 0");
    if (p->P >= ((int64_t)1 << 31)) return set_error(RR_E_SHAPE, "latent pages need P < 2^31 (int32 positions)");
    if (p->flags) return set_error(RR_E_UNSUPPORTED, "shard flags are not built for latent pages");
    if ((int64_t)p->K * p->R_max > (1 << 20)) return set_error(RR_E_SHAPE, "K*R_max too large");
    return RR_OK;
  }
  if (p->topk != 0)
    return set_error(RR_E_UNSUPPORTED, "top-k selection needs latent pages");
  if (p->d_qk != p->d_v || (p->d_qk != 64 && p->d_qk != 128))
    return set_error(RR_E_UNSUPPORTED, "dense head dims must be d_qk == d_v in {64, 128} (got %d, %d)",
                     p->d_qk, p->d_v);
  // 32-bit lane offsets of a 64-key stage of K/V rows ([P][Hkv][d] bf16 or fp32)
  if ((int64_t)p->Hkv * p->d_qk >= ((int64_t)1 << 22))
    return set_error(RR_E_SHAPE, "Hkv*d_qk must be below 2^22 (got %lld)", (long long)p->Hkv * p->d_qk);
  // 32-bit index products inside kernels: rows * heads * dims per response tensor
  const int64_t row_elems = (int64_t)p->K * p->R_max * p->Hq * (int64_t)p->d_qk;
  if (row_elems > (int64_t)1 << 31)
    return set_error(RR_E_SHAPE, "K*R_max*Hq*d_qk exceeds 2^31 elements");
  if (n_parts_of(p) > (1 << 20)) return set_error(RR_E_SHAPE, "too many prompt chunks");
  return RR_OK;
}

int64_t n_chunks_of(const rr_problem* p) { return (p->P + p->chunk - 1) / p->chunk; }

int32_t n_parts_of(const rr_problem* p) { return (int32_t)(n_chunks_of(p) + 1); }

static bool a16(const void* x) { return ((uintptr_t)x & 15u) == 0; }

static int check_aligned(const char* what, std::initializer_list<const void*> ptrs) {
  for (const void* x : ptrs)
    if (x && !a16(x)) return set_error(RR_E_SHAPE, "%s must be 16-byte aligned", what);
  return RR_OK;
}

static size_t rows_total(const rr_problem* p) { return (size_t)p->K * p->R_max * p->Hq; }

size_t ws_fwd_bytes(const rr_problem* p, bool exported) {
  if (p->latent)   // selection state and candidates (k_topk.hip)
    return topk_ws(p->P, p->topk, (size_t)p->K * p->R_max).total;
  if (exported) return 0;
  const size_t n = (size_t)n_parts_of(p) * rows_total(p);
  return align_up(n * p->d_v * sizeof(float), 256) + align_up(n * sizeof(float), 256);
}

size_t ws_pds_bytes(const rr_problem* p) {
  // response-pair P or dS, [K][R][Hq][R] bf16, plus one 128-key row segment of padding
  return align_up(((size_t)p->K * p->R_max * p->Hq * p->R_max + 128) * sizeof(uint16_t), 256);
}

size_t ws_bwd_bytes(const rr_problem* p) {
  const size_t rows = rows_total(p);
  if (p->latent)   // D, P and dS of the response pairs, chunk partials of dK_r / dV_r
    return align_up(rows * sizeof(float), 256) + 2 * ws_pds_bytes(p) +
           align_up((size_t)xty_n_chunks(p->R_max) * p->K * p->R_max * p->d_qk * sizeof(float), 256);
  // D, the dQ partials (whose region the response dK/dV partial slots reuse once dQ is
  // reduced), then (bf16) the packed row stream of the response dK/dV kernel
  const size_t dq_part = (size_t)n_parts_of(p) * rows * p->d_qk * sizeof(float);
  const size_t slots = p->dtype == RR_BF16 ? ws_dkdv_slots_bytes(p) : 0;
  return align_up(rows * sizeof(float), 256) + align_up(dq_part > slots ? dq_part : slots, 256) +
         (p->dtype == RR_BF16 ? ws_prompt_bytes(p) : 0);
}

size_t ws_dkdv_slots_bytes(const rr_problem* p) {
  return (size_t)p->K * dkdv_slots_per_response(p->R_max, p->Hkv, p->Hq / p->Hkv) * 128 * (p->d_qk + p->d_v) *
         sizeof(float);
}

// Stream rows per KV head bound for the workspace: every response at R_max rows.
static int64_t pg_rows_max(const rr_problem* p) {
  const int64_t per = ((int64_t)p->R_max * (p->Hq / p->Hkv) + 63) / 64 * 64;
  return per * p->K;
}

size_t ws_prompt_bytes(const rr_problem* p) {
  // packed Q and dO rows [Hkv][n_rows][d], then per 64-row stage lse2 and -D
  const size_t rows = (size_t)p->Hkv * pg_rows_max(p);
  const size_t esz = p->dtype == RR_BF16 ? 2 : 4;
  return 2 * align_up(rows * p->d_qk * esz, 256) + align_up(rows * 2 * sizeof(float), 256);
}

static int check_r_len(const rr_problem* p, const int32_t* r_len) {
  if (!r_len) return set_error(RR_E_NULL, "r_len is NULL");
  for (int k = 0; k < p->K; ++k)
    if (r_len[k] < 0 || r_len[k] > p->R_max)
      return set_error(RR_E_SHAPE, "r_len[%d] = %d outside [0, R_max=%d]", k, r_len[k], p->R_max);
  return RR_OK;
}

static int check_resident(const rr_problem* p, const rr_resident* kv) {
  if (!kv) return set_error(RR_E_NULL, "resident is NULL");
  if (p->P > 0 && (!kv->k_p || (!kv->v_p && !p->latent)))
    return set_error(RR_E_NULL, "resident k_p / v_p is NULL");
  if (kv->P != p->P)
    return set_error(RR_E_SHAPE, "resident P (%lld) != problem P (%lld)", (long long)kv->P,
                     (long long)p->P);
  return RR_OK;
}

int validate_fwd(const rr_problem* p, const rr_resident* kv, const void* q, const void* k_r,
                 const void* v_r, const int32_t* r_len, const float* q_idx, const float* o,
                 const float* lse, const float* part_o, const float* part_lse,
                 const int32_t* topk_idx, const void* ws, size_t ws_bytes) {
  (void)q_idx;
  int rc = validate_problem(p);
  if (rc) return rc;
  if ((rc = check_resident(p, kv))) return rc;
  if (!q || !k_r || (!v_r && !p->latent)) return set_error(RR_E_NULL, "q / k_r / v_r is NULL");
  if ((rc = check_r_len(p, r_len))) return rc;
  if (p->latent) {
    if (!q_idx || !kv->k_idx || !topk_idx) return set_error(RR_E_NULL, "q_idx / k_idx / topk_idx is NULL");
    if (!o || !lse) return set_error(RR_E_NULL, "o and lse are required for latent pages");
    if (part_o || part_lse) return set_error(RR_E_UNSUPPORTED, "partials export is not built for latent pages");
    if ((rc = check_aligned("q / k_r / latent / q_idx / k_idx / o / ws", {q, k_r, kv->k_p, q_idx, kv->k_idx, o, ws})))
      return rc;
    const size_t need = ws_fwd_bytes(p, false);
    if (!ws || ws_bytes < need)
      return set_error(RR_E_WORKSPACE, "workspace of %zu bytes needed (got %zu%s)", need, ws_bytes, ws ? "" : ", NULL");
    return RR_OK;
  }
  if ((o == nullptr) != (lse == nullptr))
    return set_error(RR_E_NULL, "o and lse must both be given or both be NULL");
  if ((part_o == nullptr) != (part_lse == nullptr))
    return set_error(RR_E_NULL, "part_o and part_lse must both be given or both be NULL");
  if (!o && !part_o) return set_error(RR_E_NULL, "no output: give o/lse, part_o/part_lse or both");
  if ((rc = check_aligned("q / k_r / v_r / k_p / v_p / o / part_o", {q, k_r, v_r, kv->k_p, kv->v_p, o, part_o})))
    return rc;
  const size_t need = ws_fwd_bytes(p, part_o != nullptr);
  if (need && (!ws || ws_bytes < need))
    return set_error(RR_E_WORKSPACE, "workspace of %zu bytes needed (got %zu%s)", need, ws_bytes,
                     ws ? "" : ", NULL");
  return RR_OK;
}

int validate_bwd(const rr_problem* p, const rr_resident* kv, const void* q, const void* k_r,
                 const void* v_r, const int32_t* r_len, const int32_t* topk_idx,
                 const float* o, const float* lse, const void* d_o, const float* dq,
                 const float* dk_r, const float* dv_r, int32_t accumulate, int32_t block_idx,
                 const void* ws, size_t ws_bytes) {
  int rc = validate_problem(p);
  if (rc) return rc;
  if ((rc = check_resident(p, kv))) return rc;
  if (!q || !k_r || (!v_r && !p->latent) || !o || !lse || !d_o)
    return set_error(RR_E_NULL, "q / k_r / v_r / o / lse / d_o is NULL");
  if (p->latent && !topk_idx) return set_error(RR_E_NULL, "topk_idx is NULL");
  const bool owns_resp = !(p->flags & RR_FLAG_SHARD_NO_RESPONSE);
  if (!dq || (owns_resp && (!dk_r || !dv_r))) return set_error(RR_E_NULL, "dq / dk_r / dv_r is NULL");
  if ((rc = check_r_len(p, r_len))) return rc;
  if (accumulate != 0 && accumulate != 1) return set_error(RR_E_SHAPE, "accumulate must be 0 or 1");
  if ((rc = check_aligned("q / k_r / v_r / k_p / v_p / o / d_o / dq / dk_r / dv_r / ws",
                          {q, k_r, v_r, kv->k_p, kv->v_p, o, d_o, dq, dk_r, dv_r, ws})))
    return rc;
  const int32_t nb = (p->R_max + p->block - 1) / p->block;
  if (block_idx < -1 || block_idx >= nb)
    return set_error(RR_E_SHAPE, "block_idx %d outside [-1, %d)", block_idx, nb);
  const size_t need = ws_bwd_bytes(p);
  if (!ws || ws_bytes < need)
    return set_error(RR_E_WORKSPACE, "workspace of %zu bytes needed (got %zu%s)", need, ws_bytes,
                     ws ? "" : ", NULL");
  return RR_OK;
}

int validate_prompt_grads(const rr_problem* p, const rr_resident* kv, const void* q,
                          const int32_t* r_len, const float* o, const float* lse, const void* d_o,
                          int64_t key_lo, int64_t key_hi, const float* dk_p, const float* dv_p,
                          int32_t accumulate, const void* ws, size_t ws_bytes) {
  int rc = validate_problem(p);
  if (rc) return rc;
  if (p->latent) return set_error(RR_E_UNSUPPORTED, "prompt gradients are built for dense K/V pages");
  if ((rc = check_resident(p, kv))) return rc;
  if (!q || !o || !lse || !d_o || !dk_p || !dv_p)
    return set_error(RR_E_NULL, "q / o / lse / d_o / dk_p / dv_p is NULL");
  if ((rc = check_r_len(p, r_len))) return rc;
  if (accumulate != 0 && accumulate != 1) return set_error(RR_E_SHAPE, "accumulate must be 0 or 1");
  if (key_lo < 0 || key_lo > key_hi || key_hi > p->P)
    return set_error(RR_E_SHAPE, "key range [%lld, %lld) outside [0, P=%lld]", (long long)key_lo,
                     (long long)key_hi, (long long)p->P);
  if ((rc = check_aligned("q / k_p / v_p / o / d_o / dk_p / dv_p / ws",
                          {q, kv->k_p, kv->v_p, o, d_o, dk_p, dv_p, ws})))
    return rc;
  if ((int64_t)p->Hkv * pg_rows_max(p) * p->d_qk > ((int64_t)1 << 31))
    return set_error(RR_E_SHAPE, "stream of K*R_max*Hq*d_qk elements exceeds 2^31");
  const size_t need = ws_prompt_bytes(p);
  if (!ws || ws_bytes < need)
    return set_error(RR_E_WORKSPACE, "workspace of %zu bytes needed (got %zu%s)", need, ws_bytes,
                     ws ? "" : ", NULL");
  return RR_OK;
}

PgGeom make_pg_geom(const rr_problem* p, const int32_t* r_len, int32_t row_lo, int32_t row_hi) {
  PgGeom pg;
  memset(&pg, 0, sizeof(pg));
  const int64_t grp = p->Hq / p->Hkv;
  pg.m_lo = (int32_t)((int64_t)row_lo * grp / 64 * 64);
  int64_t at = 0;
  for (int k = 0; k < p->K; ++k) {
    pg.off[k] = (int32_t)at;
    const int64_t m_hi = (int64_t)(r_len[k] < row_hi ? r_len[k] : row_hi) * grp;
    if (m_hi > pg.m_lo) at += (m_hi - pg.m_lo + 63) / 64 * 64;
  }
  for (int k = p->K; k <= RR_MAX_K; ++k) pg.off[k] = (int32_t)at;
  pg.n_rows = (int32_t)at;
  return pg;
}

static int blend_shape(int64_t rows, int32_t Hkv, int32_t d, int32_t dtype) {
  if (rows < 0 || Hkv < 1 || d < 8 || d % 8 != 0 || d > 4096)
    return set_error(RR_E_SHAPE, "blend needs rows >= 0, Hkv >= 1, d a multiple of 8 in [8, 4096] "
                     "(got %lld, %d, %d)", (long long)rows, Hkv, d);
  if (dtype != RR_F32 && dtype != RR_BF16) return set_error(RR_E_SHAPE, "dtype must be RR_F32 or RR_BF16");
  if (rows * Hkv * (int64_t)d > ((int64_t)1 << 40)) return set_error(RR_E_SHAPE, "blend too large");
  return RR_OK;
}

int validate_blend(int64_t rows, int32_t Hkv, int32_t d, int32_t dtype, const float* alpha,
                   const void* x_layer, const void* x_last, const void* x_out) {
  int rc = blend_shape(rows, Hkv, d, dtype);
  if (rc) return rc;
  if (!alpha || ((!x_layer || !x_last || !x_out) && rows > 0))
    return set_error(RR_E_NULL, "alpha / x_layer / x_last / x_out is NULL");
  return check_aligned("x_layer / x_last / x_out", {x_layer, x_last, x_out});
}

int validate_blend_bwd(int64_t rows, int32_t Hkv, int32_t d, int32_t dtype, const float* alpha,
                       const void* x_layer, const void* x_last, const float* d_out, const float* d_layer,
                       const float* d_last, const float* d_alpha, int32_t accumulate) {
  int rc = blend_shape(rows, Hkv, d, dtype);
  if (rc) return rc;
  if (!alpha || !d_alpha || ((!x_layer || !x_last || !d_out) && rows > 0))
    return set_error(RR_E_NULL, "alpha / d_alpha / x_layer / x_last / d_out is NULL");
  if (accumulate != 0 && accumulate != 1) return set_error(RR_E_SHAPE, "accumulate must be 0 or 1");
  return check_aligned("x_layer / x_last / d_out / d_layer / d_last", {x_layer, x_last, d_out, d_layer, d_last});
}

int validate_merge(int32_t n_parts, int64_t rows, int32_t d_v, const float* part_o,
                   const float* part_lse, const float* o, const float* lse) {
  if (n_parts < 1) return set_error(RR_E_SHAPE, "n_parts must be >= 1 (got %d)", n_parts);
  if (rows < 0) return set_error(RR_E_SHAPE, "rows must be >= 0");
  if (d_v < 1 || d_v > 4096) return set_error(RR_E_SHAPE, "d_v must be in [1, 4096] (got %d)", d_v);
  if ((int64_t)n_parts * rows * d_v > ((int64_t)1 << 40))
    return set_error(RR_E_SHAPE, "merge too large");
  if (rows > 0 && (!part_o || !part_lse || !o || !lse))
    return set_error(RR_E_NULL, "part_o / part_lse / o / lse is NULL");
  return RR_OK;
}

// Seal of a gradient tag: a 64-bit mix (splitmix64 finaliser) of the tag's fields and a
// library constant.  It tells a tag that rr_attn_bwd wrote from one that it did not
// (zero-filled, edited, assembled by hand); it is a consistency check, not a secret.
static uint64_t mix64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

uint64_t tag_seal(const rr_grad_tag* t) {
  uint64_t h = mix64(0x7272617474616731ull ^ t->version);
  h = mix64(h ^ (uint64_t)(uintptr_t)t->resident);
  return mix64(h ^ (uint64_t)t->P);
}

void write_tag(const rr_resident* kv, rr_grad_tag* t) {
  t->version = kv->version;
  t->resident = kv->k_p;
  t->P = kv->P;
  t->seal = tag_seal(t);
}

int validate_accum(const rr_accum* acc, int32_t member_g, const rr_grad_tag* tag,
                   const float* const* grads, const int64_t* n_elems) {
  if (!acc) return set_error(RR_E_NULL, "accumulator is NULL");
  if (acc->poisoned)
    return set_error(RR_E_POISONED, "the window holds part of a member after a failed launch; discard it");
  if (acc->n_bufs < 1 || acc->n_bufs > RR_MAX_ACC)
    return set_error(RR_E_SHAPE, "n_bufs must be in [1, %d] (got %d)", RR_MAX_ACC, acc->n_bufs);
  if (acc->G < 1) return set_error(RR_E_SHAPE, "G must be >= 1");
  if (!acc->seen) return set_error(RR_E_NULL, "seen mask is NULL");
  if (member_g < 0 || member_g >= acc->G)
    return set_error(RR_E_RANGE, "member %d outside [0, G=%d)", member_g, acc->G);
  if (!tag) return set_error(RR_E_NULL, "gradient tag is NULL");
  if (tag->seal != tag_seal(tag))
    return set_error(RR_E_STALE, "member %d: the gradient tag was not written by rr_attn_bwd", member_g);
  if (tag->version != acc->version)
    return set_error(RR_E_STALE, "member %d computed against resident version %llu, window is at %llu",
                     member_g, (unsigned long long)tag->version, (unsigned long long)acc->version);
  if (acc->resident && (tag->resident != acc->resident || tag->P != acc->resident_P))
    return set_error(RR_E_STALE, "member %d computed against another resident prompt state than the window's",
                     member_g);
  if (acc->seen[member_g])
    return set_error(RR_E_DUPLICATE, "member %d already accumulated in this window", member_g);
  if (!grads || !n_elems) return set_error(RR_E_NULL, "grads / n_elems is NULL");
  for (int i = 0; i < acc->n_bufs; ++i) {
    if (n_elems[i] < 0 || n_elems[i] > acc->n[i])
      return set_error(RR_E_SHAPE, "buffer %d: %lld elements exceed the accumulator's %lld", i,
                       (long long)n_elems[i], (long long)acc->n[i]);
    if (n_elems[i] > 0 && (!grads[i] || !acc->buf[i]))
      return set_error(RR_E_NULL, "buffer %d: gradient or accumulator pointer is NULL", i);
  }
  return RR_OK;
}

bool ptr_accessible(bool query_ok, PtrKind kind, bool has_device_ptr) {
  if (!query_ok) return false;
  switch (kind) {
    case PtrKind::Device:
    case PtrKind::Managed:
    case PtrKind::Unified:
      return true;
    case PtrKind::Host:        // host memory the GPU reaches only if it was pinned through HIP
      return has_device_ptr;
    default:                   // unregistered (plain host memory), arrays, unknown kinds
      return false;
  }
}

Geom make_geom(const rr_problem* p, const int32_t* r_len) {
  Geom g;
  memset(&g, 0, sizeof(g));
  g.P = p->P;
  g.chunk = p->chunk;
  g.R = p->R_max;
  g.K = p->K;
  g.Hq = p->Hq;
  g.Hkv = p->Hkv;
  g.grp = p->Hq / p->Hkv;
  g.dqk = p->d_qk;
  g.dv = p->d_v;
  g.n_chunks = (int32_t)n_chunks_of(p);
  g.n_parts = g.n_chunks + 1;
  g.row_lo = 0;
  g.row_hi = p->R_max;
  g.tau = p->tau;
  g.c2 = (float)(p->tau * 1.4426950408889634);
  g.resp_keys = (p->flags & RR_FLAG_SHARD_NO_RESPONSE) ? 0 : 1;
  for (int k = 0; k < p->K; ++k) g.r_len[k] = r_len[k];
  g.part_step = (int64_t)p->K * p->R_max * p->Hq;   // part-major unless a caller picks otherwise
  g.row_step = 1;
  return g;
}

}  // namespace rr

extern "C" {

size_t rr_workspace_bytes(const rr_problem* p, int op) {
  if (rr::validate_problem(p)) return 0;
  if (op == RR_OP_FWD) return rr::ws_fwd_bytes(p, false);
  if (op == RR_OP_BWD) return rr::ws_bwd_bytes(p);
  if (op == RR_OP_PROMPT_GRADS) {
    if (p->latent) {
      rr::set_error(RR_E_UNSUPPORTED, "prompt gradients are built for dense K/V pages");
      return 0;
    }
    return rr::ws_prompt_bytes(p);
  }
  rr::set_error(RR_E_SHAPE, "unknown op %d", op);
  return 0;
}

int32_t rr_num_parts(const rr_problem* p) {
  if (rr::validate_problem(p)) return 0;
  return rr::n_parts_of(p);
}

int rr_accum_check_complete(const rr_accum* acc) {
  if (!acc || !acc->seen) return rr::set_error(RR_E_NULL, "accumulator or seen mask is NULL");
  if (acc->poisoned)
    return rr::set_error(RR_E_POISONED, "the window holds part of a member after a failed launch; discard it");
  for (int g = 0; g < acc->G; ++g)
    if (!acc->seen[g]) return rr::set_error(RR_E_MISSING, "member %d of %d was never accumulated", g, acc->G);
  return RR_OK;
}

const char* rr_last_error(void) { return rr::last_error(); }

}  // extern "C"
