// Work split of the response-key dK/dV kernel (k_kv_grads.hip), as plain constexpr
// functions on integers: the kernels and the host launcher call them, and
// tests/native/host_checks.cpp, compiled for the host, checks that every (response, KV
// head, key tile) gets its stages cut into segments that cover them exactly once, and that
// the later segments' partial slots are distinct and within the workspace's bound.
//
// The key-parallel kernel gives a 128-key tile of response k every stream stage that holds
// a row able to see one of its keys: from the stage of row max(j0, row_lo) to the
// response's last.  Tiles near the start of a response see many more rows than tiles near
// its end; cutting each tile's run into segments of at most `seg` stages makes the work
// items of one launch cost about the same.
#pragma once

#include <stdint.h>

#include "rr_internal.h"

namespace rr {

constexpr int kPgStageRows = 64;   // stream rows per stage
constexpr int kRespKeys = 128;     // keys per response tile

// 128-key tiles of response k that the launch's rows can see.
constexpr int resp_tiles(const Geom& g, int k) {
  return ((g.r_len[k] < g.row_hi ? g.r_len[k] : g.row_hi) + kRespKeys - 1) / kRespKeys;
}

// Stream stages of tile kt of response k (at least one for every tile resp_tiles counts).
constexpr int resp_tile_stages(const Geom& g, const PgGeom& pg, int k, int kt) {
  const int n_seg = (pg.off[k + 1] - pg.off[k]) / kPgStageRows;
  const int j0 = kt * kRespKeys;
  const int s0 = ((j0 > g.row_lo ? j0 : g.row_lo) * g.grp - pg.m_lo) / kPgStageRows;
  return n_seg > s0 ? n_seg - s0 : 0;
}

// Work items: (k, KV head, tile, segment) in that order.  seg[k] is response k's segment
// length, item_off[k] its first item (Hkv times its items per KV head), slot_off[k] its
// first partial slot (one per segment after a tile's first).  A response's segments
// depend only on its own rows in the launch, never on the other responses of a call, so a
// call over K responses sums every key's gradient in the order K calls of one response
// would.
struct DkdvSplit {
  int32_t seg[RR_MAX_K];
  int32_t item_off[RR_MAX_K + 1];
  int32_t slot_off[RR_MAX_K + 1];
};

// Segments of tile kt.
constexpr int resp_tile_items(const Geom& g, const PgGeom& pg, const DkdvSplit& sp, int k, int kt) {
  return (resp_tile_stages(g, pg, k, kt) + sp.seg[k] - 1) / sp.seg[k];
}

// Position of an item of one KV head of response k (rem counts from that head's first).
struct DkdvPos {
  int kt;        // tile, -1 past the last
  int seg_idx;   // segment within the tile
  int n_items;   // the tile's segments
  int slot;      // the head's slot index of the tile's segment 1
};

constexpr DkdvPos dkdv_find(const Geom& g, const PgGeom& pg, const DkdvSplit& sp, int k, int rem) {
  DkdvPos d{-1, 0, 0, 0};
  const int nt = resp_tiles(g, k);
  int slot = 0;
  for (int kt = 0; kt < nt; ++kt) {
    const int n = resp_tile_items(g, pg, sp, k, kt);
    if (rem < n) {
      d.kt = kt;
      d.seg_idx = rem;
      d.n_items = n;
      d.slot = slot;
      return d;
    }
    rem -= n;
    slot += n - 1;
  }
  return d;
}

// Absolute slot of segment 1 of tile kt of (k, KV head gh).
constexpr int64_t dkdv_slot_base(const Geom& g, const DkdvSplit& sp, int k, int gh, int head_slot) {
  return sp.slot_off[k] + (int64_t)gh * ((sp.slot_off[k + 1] - sp.slot_off[k]) / g.Hkv) + head_slot;
}

// Slot of segment 1 of tile kt of (k, KV head gh), the one the reduction reads first.
constexpr int64_t dkdv_tile_slot(const Geom& g, const PgGeom& pg, const DkdvSplit& sp, int k, int gh, int kt) {
  int slot = 0;
  for (int t = 0; t < kt; ++t) slot += resp_tile_items(g, pg, sp, k, t) - 1;
  return dkdv_slot_base(g, sp, k, gh, slot);
}

// Work item idx of a launch: its response, KV head, tile and segment, the segment's
// stages (sequence stages [t0, t0 + n_stages) of the tile, counted down from the
// response's last stage: sequence stage t is stream stage n_top - 1 - t of the response),
// and for a later segment (seg_idx >= 1) its partial slot.  k = -1 past the last item.
struct DkdvItem {
  int k, gh, kt, seg_idx;
  int t0, n_stages, n_top;
  int64_t slot;
};

constexpr DkdvItem dkdv_item(const Geom& g, const PgGeom& pg, const DkdvSplit& sp, int idx) {
  DkdvItem it{-1, 0, 0, 0, 0, 0, 0, -1};
  int k = 0;
  while (k < g.K && idx >= sp.item_off[k + 1]) ++k;
  if (k >= g.K || idx < 0) return it;
  const int per_head = (sp.item_off[k + 1] - sp.item_off[k]) / g.Hkv;
  const DkdvPos pos = dkdv_find(g, pg, sp, k, (idx - sp.item_off[k]) % per_head);
  if (pos.kt < 0) return it;
  it.k = k;
  it.gh = (idx - sp.item_off[k]) / per_head;
  it.kt = pos.kt;
  it.seg_idx = pos.seg_idx;
  it.t0 = pos.seg_idx * sp.seg[k];
  const int left = resp_tile_stages(g, pg, k, pos.kt) - it.t0;
  it.n_stages = left < sp.seg[k] ? left : sp.seg[k];
  it.n_top = (pg.off[k + 1] - pg.off[k]) / kPgStageRows - it.t0;
  it.slot = pos.seg_idx > 0 ? dkdv_slot_base(g, sp, k, it.gh, pos.slot) + pos.seg_idx - 1 : -1;
  return it;
}

// The split of one launch: seg[k] gives about items_target later segments over response
// k's stage-tiles (never fewer than min_seg stages), so that it has at most items_target
// of them.  Returns the number of items; *n_slots the later segments, *tiles the key tiles.
constexpr int64_t plan_dkdv_split(const Geom& g, const PgGeom& pg, int items_target, int min_seg, DkdvSplit& sp,
                                  int64_t& n_slots, int64_t& tiles) {
  tiles = 0;
  int64_t items = 0;
  n_slots = 0;
  for (int k = 0; k <= RR_MAX_K; ++k) {
    sp.item_off[k] = (int32_t)items;
    sp.slot_off[k] = (int32_t)n_slots;
    if (k >= g.K) continue;
    int64_t total = 0;
    for (int kt = 0; kt < resp_tiles(g, k); ++kt) total += (int64_t)g.Hkv * resp_tile_stages(g, pg, k, kt);
    const int64_t want = (total + items_target - 1) / items_target;
    sp.seg[k] = (int32_t)(want > min_seg ? want : min_seg);
    tiles += (int64_t)g.Hkv * resp_tiles(g, k);
    int64_t it = 0;
    for (int kt = 0; kt < resp_tiles(g, k); ++kt) it += resp_tile_items(g, pg, sp, k, kt);
    items += g.Hkv * it;
    n_slots += g.Hkv * (it - resp_tiles(g, k));
  }
  return items;
}

}  // namespace rr
