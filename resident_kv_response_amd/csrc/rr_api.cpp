// C ABI entry points: validate, carve the caller's workspace, launch on the caller's
// stream.  No device memory is allocated here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <utility>
#include <string>
#include <vector>

#include "kernels.h"
#include "rr_internal.h"

namespace rr {

hipError_t launch_fwd_partials_f32(const Geom& g, const AttnPtrs& a, hipStream_t s);
hipError_t launch_fwd_partials_bf16(const Geom& g, const AttnPtrs& a, hipStream_t s);
hipError_t launch_dq_partials_f32(const Geom& g, const AttnPtrs& a, hipStream_t s);
hipError_t launch_dq_partials_bf16(const Geom& g, const AttnPtrs& a, hipStream_t s);
hipError_t launch_dkdv_f32(const Geom& g, const AttnPtrs& a, int key_hi, hipStream_t s);

hipError_t launch_fwd_partials(const Geom& g, int dtype, const AttnPtrs& a, hipStream_t s) {
  return dtype == RR_BF16 ? launch_fwd_partials_bf16(g, a, s) : launch_fwd_partials_f32(g, a, s);
}
hipError_t launch_dq_partials(const Geom& g, int dtype, const AttnPtrs& a, hipStream_t s) {
  return dtype == RR_BF16 ? launch_dq_partials_bf16(g, a, s) : launch_dq_partials_f32(g, a, s);
}
// fp32 problems; bf16 problems take the key-parallel kernel over the packed row stream
// (launch_resp_dkdv).
hipError_t launch_dkdv(const Geom& g, int dtype, const AttnPtrs& a, int key_hi, hipStream_t s) {
  (void)dtype;
  return launch_dkdv_f32(g, a, key_hi, s);
}

// ---- profiling: HIP events around every launch -----------------------------------------
namespace {

struct ProfRec {
  const char* name;
  hipEvent_t a, b;
};

struct Prof {
  std::mutex mu;
  bool on = false;
  std::vector<ProfRec> recs;
};

Prof& prof() {
  static Prof p;
  return p;
}

template <class F>
hipError_t timed(const char* name, hipStream_t s, F&& launch) {
  Prof& P = prof();
  bool on;
  {
    std::lock_guard<std::mutex> lk(P.mu);
    on = P.on;
  }
  if (!on) return launch();
  hipEvent_t a, b;
  hipError_t e = hipEventCreate(&a);
  if (e != hipSuccess) return e;
  if ((e = hipEventCreate(&b)) != hipSuccess) {
    (void)hipEventDestroy(a);
    return e;
  }
  if ((e = hipEventRecord(a, s)) != hipSuccess) {
    (void)hipEventDestroy(a);
    (void)hipEventDestroy(b);
    return e;
  }
  e = launch();
  const hipError_t e2 = hipEventRecord(b, s);
  {
    std::lock_guard<std::mutex> lk(P.mu);
    P.recs.push_back({name, a, b});
  }
  return e != hipSuccess ? e : e2;
}

int hip_fail(hipError_t e, const char* what) {
  return set_error(RR_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Every non-NULL tensor pointer must be memory the GPU can reach (device memory, or host
// memory pinned through HIP): a plain host pointer would fault inside a kernel.  Checked
// after validation, before the first launch.
PtrKind ptr_kind(hipMemoryType t) {
  switch (t) {
    case hipMemoryTypeUnregistered: return PtrKind::Unregistered;
    case hipMemoryTypeHost: return PtrKind::Host;
    case hipMemoryTypeDevice: return PtrKind::Device;
    case hipMemoryTypeManaged: return PtrKind::Managed;
    case hipMemoryTypeArray: return PtrKind::Array;
    case hipMemoryTypeUnified: return PtrKind::Unified;
    default: return PtrKind::Unknown;
  }
}

int check_dev(std::initializer_list<std::pair<const char*, const void*>> ptrs) {
  for (const auto& np : ptrs) {
    if (!np.second) continue;
    hipPointerAttribute_t a;
    memset(&a, 0, sizeof(a));
    const hipError_t e = hipPointerGetAttributes(&a, np.second);
    if (e != hipSuccess) (void)hipGetLastError();
    if (!ptr_accessible(e == hipSuccess, ptr_kind(a.type), a.devicePointer != nullptr))
      return set_error(RR_E_PTR, "%s is not memory the GPU can access", np.first);
  }
  return RR_OK;
}

float* carve(void* base, size_t offset) {
  return reinterpret_cast<float*>(static_cast<char*>(base) + offset);
}

}  // namespace

}  // namespace rr

// Workspace of rr_attn_fwd_static, for callers that cannot allocate: each GPU the library
// runs on holds its own copy (in that device's code object) until the process ends.  In
// host code `scratch` names a host-side stand-in; its device address on the current
// device comes from hipGetSymbolAddress, once per device, and only that address is used.
static __device__ __align__(256) char scratch[RR_STATIC_SCRATCH_BYTES];

namespace rr {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on the first call there).
int scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return set_error(RR_E_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    }
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return RR_OK;
}

}  // namespace

// Latent-page backward: D, then per-row dQ (which also writes the response pairs' P and dS),
// then dK_r = tau dS^T Q and dV_r = P^T dO over the query rows of each block, last block
// first.
int latent_bwd(const rr_problem* p, const rr_resident* kv, const void* q, const void* k_r,
               const int32_t* r_len, const int32_t* topk_idx, const float* o, const float* lse,
               const void* d_o, float* dq, float* dk_r, float* dv_r, int32_t accumulate,
               int32_t block_idx, void* ws, hipStream_t s) {
  Geom g = make_geom(p, r_len);
  const size_t rows = (size_t)p->K * p->R_max * p->Hq;
  float* Dvec = carve(ws, 0);
  uint16_t* p_r = reinterpret_cast<uint16_t*>(carve(ws, align_up(rows * sizeof(float), 256)));
  uint16_t* ds_r = reinterpret_cast<uint16_t*>(carve(ws, align_up(rows * sizeof(float), 256) + ws_pds_bytes(p)));
  float* part = carve(ws, align_up(rows * sizeof(float), 256) + 2 * ws_pds_bytes(p));
  const int nb = (p->R_max + p->block - 1) / p->block;
  if (block_idx >= 0) {
    g.row_lo = block_idx * p->block;
    g.row_hi = std::min(p->R_max, g.row_lo + p->block);
  }
  hipError_t e;
  if ((e = timed("bwd_pre", s, [&] { return launch_bwd_pre(g, p->dtype, o, d_o, Dvec, s); })))
    return hip_fail(e, "bwd_pre");
  if ((e = timed("sparse_dq", s, [&] {
         return launch_sparse_dq(g, p->topk, q, kv->k_p, k_r, topk_idx, d_o, lse, Dvec, dq, p_r, ds_r,
                                 accumulate, s);
       })))
    return hip_fail(e, "sparse_dq");
  if (!accumulate) {
    if ((e = timed("zero_rows", s, [&] {
           hipError_t e1 = launch_zero_rows(dk_r, p->K, p->R_max, 0, g.row_hi, p->d_qk, s);
           return e1 != hipSuccess ? e1 : launch_zero_rows(dv_r, p->K, p->R_max, 0, g.row_hi, p->d_v, s);
         })))
      return hip_fail(e, "zero_rows");
  }
  const int b_hi = block_idx >= 0 ? block_idx : nb - 1;
  const int b_lo = block_idx >= 0 ? block_idx : 0;
  for (int b = b_hi; b >= b_lo; --b) {   // reverse block walk
    const int lo = b * p->block, hi = std::min(p->R_max, lo + p->block);
    if ((e = timed("xty_dk", s, [&] {
           return launch_xty(ds_r, static_cast<const uint16_t*>(q), p->d_qk, p->d_qk, dk_r, p->d_qk, part, g,
                             lo, hi, hi, p->tau, s);
         })))
      return hip_fail(e, "xty_dk");
    if ((e = timed("xty_dv", s, [&] {
           return launch_xty(p_r, static_cast<const uint16_t*>(d_o), p->d_v, p->d_v, dv_r, p->d_v, part, g,
                             lo, hi, hi, 1.0f, s);
         })))
      return hip_fail(e, "xty_dv");
  }
  return RR_OK;
}

}  // namespace rr

using namespace rr;

extern "C" {

int rr_attn_fwd(const rr_problem* p, const rr_resident* kv, const void* q, const void* k_r,
                const void* v_r, const int32_t* r_len, const float* q_idx, float* o, float* lse,
                float* part_o, float* part_lse, int32_t* topk_idx, void* ws, size_t ws_bytes,
                void* stream) {
  clear_error();
  return rr_attn_fwd_impl(p, kv, q, k_r, v_r, r_len, q_idx, o, lse, part_o, part_lse, topk_idx, ws, ws_bytes,
                          stream, false);
}

int rr_attn_fwd_static(const rr_problem* p, const rr_resident* kv, const void* q, const void* k_r,
                       const void* v_r, const int32_t* r_len, const float* q_idx, float* o, float* lse,
                       float* part_o, float* part_lse, int32_t* topk_idx, void* stream) {
  clear_error();
  // every argument check first, against a stand-in workspace of the scratch's size, so an
  // invalid call touches no device state
  int rc = validate_fwd(p, kv, q, k_r, v_r, r_len, q_idx, o, lse, part_o, part_lse, topk_idx,
                        reinterpret_cast<void*>(static_cast<uintptr_t>(256)), RR_STATIC_SCRATCH_BYTES);
  if (rc == RR_E_WORKSPACE)
    return set_error(RR_E_WORKSPACE, "the problem needs %zu bytes of workspace; the static scratch holds %zu",
                     ws_fwd_bytes(p, part_o != nullptr), (size_t)RR_STATIC_SCRATCH_BYTES);
  if (rc) return rc;
  void* ws = nullptr;
  if ((rc = scratch_ptr(&ws))) return rc;
  return rr_attn_fwd_impl(p, kv, q, k_r, v_r, r_len, q_idx, o, lse, part_o, part_lse, topk_idx, ws,
                          RR_STATIC_SCRATCH_BYTES, stream, true);
}

}  // extern "C"

namespace rr {

int rr_attn_fwd_impl(const rr_problem* p, const rr_resident* kv, const void* q, const void* k_r,
                     const void* v_r, const int32_t* r_len, const float* q_idx, float* o, float* lse,
                     float* part_o, float* part_lse, int32_t* topk_idx, void* ws, size_t ws_bytes,
                     void* stream, bool ws_is_scratch) {
  int rc = validate_fwd(p, kv, q, k_r, v_r, r_len, q_idx, o, lse, part_o, part_lse, topk_idx, ws,
                        ws_bytes);
  if (rc) return rc;
  // the static scratch is the library's own device memory: not looked up
  if ((rc = check_dev({{"k_p", kv->k_p}, {"v_p", kv->v_p}, {"k_idx", kv->k_idx}, {"q", q}, {"k_r", k_r},
                        {"v_r", v_r}, {"q_idx", q_idx}, {"o", o}, {"lse", lse}, {"part_o", part_o},
                        {"part_lse", part_lse}, {"topk_idx", topk_idx}, {"ws", ws_is_scratch ? nullptr : ws}})))
    return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Geom g = make_geom(p, r_len);
  const size_t rows = (size_t)p->K * p->R_max * p->Hq;
  if (p->latent) {
    // exact top-k per row (screen + candidates + exact selection) -> attention over the
    // selection + causal rows
    hipError_t e = timed("topk_select", s, [&] {
      return launch_topk(q_idx, kv->k_idx, ws, p->P, p->topk, g, topk_idx, s);
    });
    if (e != hipSuccess) return hip_fail(e, "topk_select");
    if ((e = timed("sparse_fwd", s, [&] {
           return launch_sparse_fwd(g, p->topk, q, kv->k_p, k_r, topk_idx, o, lse, s);
         })))
      return hip_fail(e, "sparse_fwd");
    return RR_OK;
  }
  float* po = part_o;
  float* pl = part_lse;
  if (!po) {   // partials in the workspace: row-major; an export buffer keeps part-major
    po = carve(ws, 0);
    pl = carve(ws, align_up((size_t)g.n_parts * rows * p->d_v * sizeof(float), 256));
    set_parts_row_major(g);
  }
  AttnPtrs a{};
  a.q = q;
  a.k_p = kv->k_p;
  a.v_p = kv->v_p;
  a.k_r = k_r;
  a.v_r = v_r;
  a.part_o = po;
  a.part_lse = pl;
  hipError_t e = timed("fwd_partials", s, [&] { return launch_fwd_partials(g, p->dtype, a, s); });
  if (e != hipSuccess) return hip_fail(e, "fwd_partials");
  if (o) {
    e = timed("lse_merge", s, [&] {
      return launch_merge(g.n_parts, (int64_t)rows, p->d_v, po, pl, o, lse, &g, s);
    });
    if (e != hipSuccess) return hip_fail(e, "lse_merge");
  }
  return RR_OK;
}

}  // namespace rr

extern "C" {

int rr_lse_merge(int32_t n_parts, int64_t rows, int32_t d_v, const float* part_o,
                 const float* part_lse, float* o, float* lse, void* stream) {
  clear_error();
  int rc = validate_merge(n_parts, rows, d_v, part_o, part_lse, o, lse);
  if (rc) return rc;
  if ((rc = check_dev({{"part_o", part_o}, {"part_lse", part_lse}, {"o", o}, {"lse", lse}}))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = timed("lse_merge", s, [&] {
    return launch_merge(n_parts, rows, d_v, part_o, part_lse, o, lse, nullptr, s);
  });
  if (e != hipSuccess) return hip_fail(e, "lse_merge");
  return RR_OK;
}

int rr_attn_bwd(const rr_problem* p, const rr_resident* kv, const void* q, const void* k_r,
                const void* v_r, const int32_t* r_len, const int32_t* topk_idx, const float* o,
                const float* lse, const void* d_o, float* dq, float* dk_r, float* dv_r,
                int32_t accumulate, int32_t block_idx, void* ws, size_t ws_bytes, rr_grad_tag* tag,
                void* stream) {
  clear_error();
  int rc = rr_attn_bwd_impl(p, kv, q, k_r, v_r, r_len, topk_idx, o, lse, d_o, dq, dk_r, dv_r, accumulate,
                            block_idx, ws, ws_bytes, stream);
  if (rc == RR_OK && tag) write_tag(kv, tag);
  return rc;
}

}  // extern "C"

namespace rr {

int rr_attn_bwd_impl(const rr_problem* p, const rr_resident* kv, const void* q, const void* k_r,
                     const void* v_r, const int32_t* r_len, const int32_t* topk_idx, const float* o,
                     const float* lse, const void* d_o, float* dq, float* dk_r, float* dv_r,
                     int32_t accumulate, int32_t block_idx, void* ws, size_t ws_bytes, void* stream) {
  int rc = validate_bwd(p, kv, q, k_r, v_r, r_len, topk_idx, o, lse, d_o, dq, dk_r, dv_r, accumulate,
                        block_idx, ws, ws_bytes);
  if (rc) return rc;
  if ((rc = check_dev({{"k_p", kv->k_p}, {"v_p", kv->v_p}, {"q", q}, {"k_r", k_r}, {"v_r", v_r},
                        {"topk_idx", topk_idx}, {"o", o}, {"lse", lse}, {"d_o", d_o}, {"dq", dq},
                        {"dk_r", dk_r}, {"dv_r", dv_r}, {"ws", ws}})))
    return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Geom g = make_geom(p, r_len);
  set_parts_row_major(g);   // the dQ partials live in the workspace
  const size_t rows = (size_t)p->K * p->R_max * p->Hq;
  if (p->latent) return latent_bwd(p, kv, q, k_r, r_len, topk_idx, o, lse, d_o, dq, dk_r, dv_r,
                                   accumulate, block_idx, ws, s);
  float* Dvec = carve(ws, 0);
  float* dq_part = carve(ws, align_up(rows * sizeof(float), 256));
  AttnPtrs a{};
  a.q = q;
  a.k_p = kv->k_p;
  a.v_p = kv->v_p;
  a.k_r = k_r;
  a.v_r = v_r;
  a.d_o = d_o;
  a.lse = lse;
  a.Dvec = Dvec;
  a.dq_part = dq_part;
  a.dk_r = dk_r;
  a.dv_r = dv_r;
  const int nb = (p->R_max + p->block - 1) / p->block;
  const int64_t kv_row = (int64_t)p->Hkv * p->d_qk;
  if (block_idx >= 0) {
    g.row_lo = block_idx * p->block;
    g.row_hi = std::min(p->R_max, g.row_lo + p->block);
  }
  hipError_t e;
  if ((e = timed("bwd_pre", s, [&] { return launch_bwd_pre(g, p->dtype, o, d_o, Dvec, s); })))
    return hip_fail(e, "bwd_pre");
  if ((e = timed("dq_partials", s, [&] { return launch_dq_partials(g, p->dtype, a, s); })))
    return hip_fail(e, "dq_partials");
  if ((e = timed("dq_reduce", s, [&] { return launch_dq_reduce(g, dq_part, dq, accumulate, s); })))
    return hip_fail(e, "dq_reduce");
  const int key_top = g.row_hi;   // response keys reachable from the launch's rows
  if (!g.resp_keys) return RR_OK;  // another shard owns the response keys and their grads
  if (!accumulate) {
    if ((e = timed("zero_rows", s, [&] {
           hipError_t e1 = launch_zero_rows(dk_r, p->K, p->R_max, 0, key_top, kv_row, s);
           return e1 != hipSuccess ? e1 : launch_zero_rows(dv_r, p->K, p->R_max, 0, key_top, kv_row, s);
         })))
      return hip_fail(e, "zero_rows");
  }
  if (p->dtype == RR_BF16) {
    // Key-parallel over the packed stream of the launch's rows [g.row_lo, g.row_hi): the
    // whole walk (block_idx = -1) in one launch, each key's gradient over every row that
    // sees it (the sum the walk forms block by block), or one block of the caller's walk.
    const PgGeom pg = make_pg_geom(p, r_len, g.row_lo, g.row_hi);
    const size_t srows = (size_t)p->Hkv * pg.n_rows;
    const size_t sbytes = align_up(srows * p->d_qk * 2, 256);
    const size_t dq_bytes = (size_t)n_parts_of(p) * rows * p->d_qk * sizeof(float);
    const size_t slot_bytes = ws_dkdv_slots_bytes(p);
    char* sbase = reinterpret_cast<char*>(carve(ws, align_up(rows * sizeof(float), 256) +
                                                        align_up(std::max(dq_bytes, slot_bytes), 256)));
    void* qs = sbase;
    void* os = sbase + sbytes;
    float* sts = reinterpret_cast<float*>(sbase + 2 * sbytes);
    // the dQ partials are reduced by now: their region holds the dK/dV partial slots
    float* slots = dq_part;
    if ((e = timed("pg_pack", s, [&] { return launch_pg_pack(g, pg, p->dtype, q, o, lse, d_o, qs, os, sts, s); })))
      return hip_fail(e, "pg_pack");
    if ((e = timed("dkdv", s, [&] {
           return launch_resp_dkdv(g, pg, k_r, v_r, qs, os, sts, slots, dk_r, dv_r, s);
         })))
      return hip_fail(e, "dkdv");
    return RR_OK;
  }
  const int b_hi = block_idx >= 0 ? block_idx : nb - 1;
  const int b_lo = block_idx >= 0 ? block_idx : 0;
  for (int b = b_hi; b >= b_lo; --b) {   // reverse block walk
    Geom gb = g;
    gb.row_lo = b * p->block;
    gb.row_hi = std::min(p->R_max, gb.row_lo + p->block);
    if ((e = timed("dkdv", s, [&] { return launch_dkdv(gb, p->dtype, a, gb.row_hi, s); })))
      return hip_fail(e, "dkdv");
  }
  return RR_OK;
}

}  // namespace rr

extern "C" {

int rr_attn_prompt_grads(const rr_problem* p, const rr_resident* kv, const void* q, const int32_t* r_len,
                         const float* o, const float* lse, const void* d_o, int64_t key_lo, int64_t key_hi,
                         float* dk_p, float* dv_p, int32_t accumulate, void* ws, size_t ws_bytes,
                         void* stream) {
  clear_error();
  int rc = validate_prompt_grads(p, kv, q, r_len, o, lse, d_o, key_lo, key_hi, dk_p, dv_p, accumulate, ws,
                                 ws_bytes);
  if (rc) return rc;
  if ((rc = check_dev({{"k_p", kv->k_p}, {"v_p", kv->v_p}, {"q", q}, {"o", o}, {"lse", lse}, {"d_o", d_o},
                        {"dk_p", dk_p}, {"dv_p", dv_p}, {"ws", ws}})))
    return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Geom g = make_geom(p, r_len);
  const PgGeom pg = make_pg_geom(p, r_len, 0, p->R_max);
  const size_t rows = (size_t)p->Hkv * pg.n_rows;
  const size_t esz = p->dtype == RR_BF16 ? 2 : 4;
  const size_t rows_bytes = align_up(rows * p->d_qk * esz, 256);
  void* qs = ws;
  void* os = carve(ws, rows_bytes);
  float* sts = carve(ws, 2 * rows_bytes);
  hipError_t e;
  if ((e = timed("pg_pack", s, [&] { return launch_pg_pack(g, pg, p->dtype, q, o, lse, d_o, qs, os, sts, s); })))
    return hip_fail(e, "pg_pack");
  if ((e = timed("prompt_dkdv", s, [&] {
         return launch_prompt_dkdv(g, pg, p->dtype, kv->k_p, kv->v_p, qs, os, sts, key_lo, key_hi, dk_p, dv_p,
                                   accumulate, s);
       })))
    return hip_fail(e, "prompt_dkdv");
  return RR_OK;
}

int rr_lastkv_blend(int64_t rows, int32_t Hkv, int32_t d, int32_t dtype, const float* alpha, const void* x_layer,
                    const void* x_last, void* x_out, void* stream) {
  clear_error();
  int rc = validate_blend(rows, Hkv, d, dtype, alpha, x_layer, x_last, x_out);
  if (rc) return rc;
  if ((rc = check_dev({{"alpha", alpha}, {"x_layer", x_layer}, {"x_last", x_last}, {"x_out", x_out}}))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = timed("lastkv_blend", s, [&] {
    return launch_lastkv_blend(rows, Hkv, d, dtype, alpha, x_layer, x_last, x_out, s);
  });
  return e != hipSuccess ? hip_fail(e, "lastkv_blend") : RR_OK;
}

int rr_lastkv_blend_bwd(int64_t rows, int32_t Hkv, int32_t d, int32_t dtype, const float* alpha,
                        const void* x_layer, const void* x_last, const float* d_out, float* d_layer,
                        float* d_last, float* d_alpha, int32_t accumulate, void* stream) {
  clear_error();
  int rc = validate_blend_bwd(rows, Hkv, d, dtype, alpha, x_layer, x_last, d_out, d_layer, d_last, d_alpha,
                              accumulate);
  if (rc) return rc;
  if ((rc = check_dev({{"alpha", alpha}, {"x_layer", x_layer}, {"x_last", x_last}, {"d_out", d_out},
                        {"d_layer", d_layer}, {"d_last", d_last}, {"d_alpha", d_alpha}})))
    return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = timed("lastkv_blend_bwd", s, [&] {
    return launch_lastkv_blend_bwd(rows, Hkv, d, dtype, alpha, x_layer, x_last, d_out, d_layer, d_last, d_alpha,
                                   accumulate, s);
  });
  return e != hipSuccess ? hip_fail(e, "lastkv_blend_bwd") : RR_OK;
}

int rr_grad_accum(rr_accum* acc, int32_t member_g, const rr_grad_tag* tag, const float* const* grads,
                  const int64_t* n_elems, float scale, void* stream) {
  clear_error();
  int rc = validate_accum(acc, member_g, tag, grads, n_elems);
  if (rc) return rc;
  for (int i = 0; i < acc->n_bufs; ++i)
    if ((rc = check_dev({{"accumulator buffer", acc->buf[i]}, {"grad", grads[i]}}))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int i = 0; i < acc->n_bufs; ++i) {
    hipError_t e = timed("grad_accum", s, [&] { return launch_axpy(acc->buf[i], grads[i], n_elems[i], scale, s); });
    if (e != hipSuccess) {
      if (i == 0) return hip_fail(e, "grad_accum");
      // buffers 0 .. i-1 already hold this member: no retry can make the window whole
      acc->poisoned = 1;
      return set_error(RR_E_POISONED, "grad_accum: launch for buffer %d failed after %d buffers were added (%s); "
                       "the window is poisoned", i, i, hipGetErrorString(e));
    }
  }
  if (!acc->resident) {
    acc->resident = tag->resident;
    acc->resident_P = tag->P;
  }
  acc->seen[member_g] = 1;
  return RR_OK;
}

int rr_profile_begin(void) {
  clear_error();
  Prof& P = prof();
  std::lock_guard<std::mutex> lk(P.mu);
  for (auto& r : P.recs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  P.recs.clear();
  P.on = true;
  return RR_OK;
}

int rr_profile_end(rr_profile_entry* out, int32_t max_entries, int32_t* n_out) {
  clear_error();
  Prof& P = prof();
  std::vector<ProfRec> recs;
  {
    std::lock_guard<std::mutex> lk(P.mu);
    P.on = false;
    recs.swap(P.recs);
  }
  std::vector<rr_profile_entry> agg;
  int rc = RR_OK;
  for (auto& r : recs) {
    float ms = 0.0f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess && rc == RR_OK) rc = hip_fail(e, "profile events");
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
    size_t i = 0;
    while (i < agg.size() && strcmp(agg[i].name, r.name) != 0) ++i;
    if (i == agg.size()) {
      rr_profile_entry z;
      memset(&z, 0, sizeof(z));
      strncpy(z.name, r.name, sizeof(z.name) - 1);
      agg.push_back(z);
    }
    agg[i].launches += 1;
    agg[i].total_ms += ms;
  }
  const int n = (int)agg.size() < max_entries ? (int)agg.size() : max_entries;
  if (out)
    for (int i = 0; i < n; ++i) out[i] = agg[i];
  if (n_out) *n_out = n;
  return rc;
}

}  // extern "C"
