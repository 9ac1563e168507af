// Host-compiled checks of the library's integer and host logic (no GPU): the address
// arithmetic of the direct global->LDS loads (csrc/k_addr.h, the functions the kernels
// call), the work split of the response dK/dV kernel (csrc/k_split.h), the
// classification of pointer lookups, and the accumulation window's
// version/resident checks (csrc/rr_validate.cpp).  Built and run by
// tests/test_host_native.py; prints one line per group and exits non-zero on the first
// failure.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <utility>
#include <vector>

#include "k_addr.h"
#include "k_split.h"
#include "rr_internal.h"

using namespace rr;

static int g_fail = 0;
#define CHECK(cond, ...)                                   \
  do {                                                     \
    if (!(cond)) {                                         \
      if (g_fail++ < 20) {                                 \
        std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
        std::fprintf(stderr, __VA_ARGS__);                 \
        std::fprintf(stderr, "\n");                        \
      }                                                    \
    }                                                      \
  } while (0)

// ---- direct loads of the ring kernels ----------------------------------------------------
// Tile shapes the kernels instantiate: forward and dQ (64-key stages, 8 waves), the
// key-parallel K/V-gradient kernels (64-row stream stages, 4 waves).
struct RowsShape { int D, n_rows, waves; };

// slack: bytes past the last valid row that a load may touch (a row wider than the stride
// runs into the next rows; the buffer ends in that much padding).
static void check_rows_shape(const RowsShape& sh, uint32_t stride, uint32_t slack = 0) {
  const int G = sh.D / 8, RPI = 64 / G, ROW = sh.D * 2;
  const int per_wave = sh.n_rows * G / (64 * sh.waves);
  CHECK(per_wave * 64 * sh.waves == sh.n_rows * G, "tile does not split over the waves");
  // the 32-bit lane offsets of the largest stage must not wrap
  CHECK((uint64_t)sh.n_rows * stride < (1ull << 31), "stride %u too large for 32-bit offsets", stride);
  for (int rows_valid = 1; rows_valid <= sh.n_rows; ++rows_valid) {
    std::vector<int> written((size_t)sh.n_rows * G, 0);
    for (int wave = 0; wave < sh.waves; ++wave)
      for (int lane = 0; lane < 64; ++lane) {
        const RowsLoadPre p = rows_load_pre(sh.D, sh.n_rows, sh.waves, wave, lane);
        for (int i = 0; i < per_wave; ++i) {
          const RowsLoadAt a = rows_load_at(p, sh.D, i, rows_valid, stride);
          const uint32_t lds = a.lds_base + 16u * (uint32_t)lane;
          const int t_row = (int)(lds / ROW), pos = (int)(lds % ROW) / 16;
          CHECK(lds % 16 == 0 && t_row < sh.n_rows, "LDS byte %u outside the tile", lds);
          CHECK(t_row == a.tile_row, "lane lands in row %d, address says %d", t_row, a.tile_row);
          written[(size_t)t_row * G + pos] += 1;
          // source: the tile row itself while it exists, else the last existing row
          const int want_row = t_row < rows_valid ? t_row : rows_valid - 1;
          CHECK(a.src_row == want_row, "rows_valid %d: tile row %d reads row %d", rows_valid, t_row, a.src_row);
          const uint64_t exact = (uint64_t)a.src_row * stride + (uint64_t)((pos ^ swz(sh.D, t_row)) * 16);
          CHECK(a.src_off == exact, "offset %u != %llu (D %d row %d pos %d)", a.src_off,
                (unsigned long long)exact, sh.D, t_row, pos);
          CHECK((uint64_t)a.src_off + 16 <= (uint64_t)rows_valid * stride + slack, "load past the stage's rows");
          (void)RPI;
        }
      }
    for (size_t k = 0; k < written.size(); ++k)
      CHECK(written[k] == 1, "granule %zu written %d times", k, written[k]);
  }
}

// Stage counts of a part of n_keys keys: every stage that is issued has rows_valid >= 1.
static void check_stages(int64_t n_keys, int BN) {
  const int64_t n_stages = (n_keys + BN - 1) / BN;
  for (int64_t s : {(int64_t)0, n_stages - 2, n_stages - 1}) {
    if (s < 0 || s >= n_stages) continue;
    const int64_t rows = n_keys - s * BN;
    CHECK(rows >= 1, "n_keys %lld stage %lld: rows_valid %lld", (long long)n_keys, (long long)s, (long long)rows);
  }
}

// ---- general tile loads (response-pair GEMM) -----------------------------------------------
// `slack`: bytes readable past row_end * stride.  The X operand (P or dS of the response
// pairs, rows of R bf16) is read in 128-column tiles from column j0, so a short row's tile
// runs into the next row and the last one into the 128-element pad that ends the buffer.
static void check_tile_shape(int D, int n_rows, int waves, int64_t stride, int64_t row_end, int64_t slack) {
  const int G = D / 8, ROW = D * 2;
  const int per_wave = n_rows * G / (64 * waves);
  for (int64_t src_row0 : {(int64_t)0, row_end - n_rows, row_end - 1, row_end / 2}) {
    if (src_row0 < 0 || src_row0 >= row_end) continue;
    const bool full = src_row0 + n_rows <= row_end;
    std::vector<int> written((size_t)n_rows * G, 0);
    for (int wave = 0; wave < waves; ++wave)
      for (int lane = 0; lane < 64; ++lane) {
        const TileLoadPre p = tile_load_pre(D, n_rows, waves, wave, lane, stride);
        for (int i = 0; i < per_wave; ++i) {
          const TileLoadAt a = tile_load_at(p, D, i, src_row0, row_end, stride, full);
          const uint32_t lds = a.lds_base + 16u * (uint32_t)lane;
          const int t_row = (int)(lds / ROW), pos = (int)(lds % ROW) / 16;
          CHECK(t_row < n_rows, "LDS byte outside the tile");
          written[(size_t)t_row * G + pos] += 1;
          const int64_t want = src_row0 + t_row < row_end ? src_row0 + t_row : row_end - 1;
          CHECK(a.src_row == want, "tile row %d reads row %lld, expected %lld", t_row, (long long)a.src_row,
                (long long)want);
          const int64_t exact = a.src_row * stride + (int64_t)((pos ^ swz(D, t_row)) * 16);
          CHECK(a.src_off == exact, "tile offset %lld != %lld", (long long)a.src_off, (long long)exact);
          CHECK(a.src_off >= 0 && a.src_off + 16 <= row_end * stride + slack,
                "tile load outside the stream: D %d stride %lld row_end %lld row %lld off %lld", D,
                (long long)stride, (long long)row_end, (long long)a.src_row, (long long)a.src_off);
        }
      }
    for (size_t k = 0; k < written.size(); ++k) CHECK(written[k] == 1, "tile granule %zu written %d times", k, written[k]);
  }
}

static void check_addresses() {
  // forward / dQ: K/V rows of one KV head, stride Hkv * D * 2 bytes ([P][Hkv][D] bf16);
  // head counts of every workload, and the largest the validation admits (Hkv*D < 2^22)
  for (int D : {64, 128}) {
    for (int hkv : {1, 2, 3, 4, 6, 8, 16, 64, 1024, (1 << 22) / D - 1}) {
      check_rows_shape({D, 64, 8}, (uint32_t)(hkv * D * 2));
    }
    // K/V-gradient kernels: packed stream rows of D bf16
    check_rows_shape({D, 64, 4}, (uint32_t)(D * 2));
  }
  // response-pair GEMM of the latent variant (ring form): 32- or 64-row stages of X rows of
  // R bf16 (128 keys) and of Y rows of 576 or 512 dims (64-dim halves)
  // (rows of fewer than 128 keys run into the next rows; the P / dS buffers end in one
  // 128-key row segment of padding)
  for (int rows : {32, 64}) {
    for (uint32_t R : {32u, 64u, 96u, 4096u, 8192u, 65536u}) check_rows_shape({128, rows, 4}, R * 2, 256);
    check_rows_shape({64, rows, 4}, 576 * 2);
    check_rows_shape({64, rows, 4}, 512 * 2);
  }
  // part lengths: chunks and remainders of the workloads, response lengths, every small count
  for (int64_t n = 1; n <= 5000; ++n) check_stages(n, 64);
  for (int64_t n : {(int64_t)8192, (int64_t)16384, (int64_t)65536, (int64_t)131072, (int64_t)1 << 20,
                    (int64_t)16778216 % (1 << 20), (int64_t)2097152})
    check_stages(n, 64);
  // response-pair GEMM of the latent variant: X rows of R bf16 (R up to 8192), Y rows of
  // 576 or 512 dims
  for (int64_t R : {(int64_t)32, (int64_t)64, (int64_t)96, (int64_t)4096, (int64_t)8192}) {
    check_tile_shape(128, 32, 4, R * 2, 64 * R, 256);
    check_tile_shape(64, 32, 4, 576 * 2, 64 * R, 0);
    check_tile_shape(64, 32, 4, 512 * 2, 64 * R, 0);
  }
  // the clamped (partial) form over a ragged end
  check_tile_shape(128, 32, 4, 256, 45, 0);
  check_tile_shape(64, 32, 4, 1152, 33, 0);
  std::printf("addresses: ok\n");
}

// ---- pointer classification ------------------------------------------------------------------
static void check_pointers() {
  CHECK(!ptr_accessible(false, PtrKind::Device, true), "failed lookup accepted");
  CHECK(!ptr_accessible(true, PtrKind::Unregistered, false), "plain host memory accepted");
  CHECK(!ptr_accessible(true, PtrKind::Unregistered, true), "unregistered memory accepted");
  CHECK(!ptr_accessible(true, PtrKind::Host, false), "host memory without a device mapping accepted");
  CHECK(ptr_accessible(true, PtrKind::Host, true), "pinned host memory refused");
  CHECK(ptr_accessible(true, PtrKind::Device, true), "device memory refused");
  CHECK(ptr_accessible(true, PtrKind::Managed, true), "managed memory refused");
  CHECK(ptr_accessible(true, PtrKind::Unified, true), "unified memory refused");
  CHECK(!ptr_accessible(true, PtrKind::Array, true), "array memory accepted");
  CHECK(!ptr_accessible(true, PtrKind::Unknown, true), "unknown memory kind accepted");
  std::printf("pointers: ok\n");
}

// ---- accumulation window -------------------------------------------------------------------
static void check_accum() {
  static float fake_buf[4], fake_grad[4];
  uint8_t seen[8] = {0};
  rr_accum acc;
  std::memset(&acc, 0, sizeof(acc));
  acc.n_bufs = 1;
  acc.buf[0] = fake_buf;
  acc.n[0] = 4;
  acc.G = 8;
  acc.version = 3;
  acc.seen = seen;
  const float* grads[1] = {fake_grad};
  const int64_t n[1] = {4};
  int k_a = 0, k_b = 0;
  rr_resident kv_a{&k_a, &k_a, nullptr, 100, 3};
  rr_resident kv_b{&k_b, &k_b, nullptr, 100, 3};   // another prompt group, same version
  rr_resident kv_new{&k_a, &k_a, nullptr, 100, 4}; // the same state under a newer version
  rr_grad_tag t_a, t_b, t_new;
  write_tag(&kv_a, &t_a);
  write_tag(&kv_b, &t_b);
  write_tag(&kv_new, &t_new);
  CHECK(validate_accum(&acc, 0, &t_a, grads, n) == RR_OK, "valid member refused");
  CHECK(validate_accum(&acc, 0, nullptr, grads, n) == RR_E_NULL, "NULL tag accepted");
  CHECK(validate_accum(&acc, 0, &t_new, grads, n) == RR_E_STALE, "other version accepted");
  rr_grad_tag forged;
  std::memset(&forged, 0, sizeof(forged));
  forged.version = 3;
  forged.resident = &k_a;
  forged.P = 100;
  CHECK(validate_accum(&acc, 0, &forged, grads, n) == RR_E_STALE, "unsealed tag accepted");
  rr_grad_tag edited = t_new;
  edited.version = 3;   // relabelled without a backward
  CHECK(validate_accum(&acc, 0, &edited, grads, n) == RR_E_STALE, "edited tag accepted");
  // the window binds to the first accepted member's resident (what rr_grad_accum records)
  acc.resident = t_a.resident;
  acc.resident_P = t_a.P;
  seen[0] = 1;
  CHECK(validate_accum(&acc, 1, &t_b, grads, n) == RR_E_STALE, "other prompt group accepted");
  CHECK(validate_accum(&acc, 1, &t_a, grads, n) == RR_OK, "same resident refused");
  CHECK(validate_accum(&acc, 0, &t_a, grads, n) == RR_E_DUPLICATE, "retry accepted");
  CHECK(validate_accum(&acc, 8, &t_a, grads, n) == RR_E_RANGE, "member 8 of 8 accepted");
  acc.poisoned = 1;
  CHECK(validate_accum(&acc, 1, &t_a, grads, n) == RR_E_POISONED, "poisoned window accepted");
  CHECK(rr_accum_check_complete(&acc) == RR_E_POISONED, "poisoned window reported complete");
  std::printf("accumulator: ok\n");
}

// ---- work split of the response dK/dV kernel --------------------------------------------
// Every (response, KV head, key tile) gets its stages [0, resp_tile_stages) from exactly one
// segment each, in order; each item's stream stages lie inside the response's stream and
// its 64-row stages hold rows that can see the tile (stage >= the one of row max(j0,
// row_lo)); later segments get distinct slots below the workspace's bound, numbered as the
// reduction reads them; and the grid's items after the last decode to nothing.
static void check_dkdv_case(int K, const std::vector<int>& lens, int R_max, int Hq, int Hkv, int row_lo,
                            int row_hi) {
  rr_problem p{};
  p.P = 4096;
  p.chunk = 1024;
  p.R_max = R_max;
  p.K = K;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.d_qk = p.d_v = 128;
  p.block = 2048;
  p.dtype = RR_BF16;
  p.tau = 0.088f;
  Geom g = make_geom(&p, lens.data());
  g.row_lo = row_lo;
  g.row_hi = row_hi;
  const PgGeom pg = make_pg_geom(&p, lens.data(), row_lo, row_hi);
  DkdvSplit sp{};
  int64_t n_slots = 0, tiles = 0;
  const int64_t items = plan_dkdv_split(g, pg, kDkdvItemsTarget, kDkdvMinSeg, sp, n_slots, tiles);
  CHECK(n_slots <= (int64_t)K * kDkdvItemsTarget &&
            n_slots <= (int64_t)K * dkdv_slots_per_response(R_max, Hkv, Hq / Hkv),
        "%lld slots", (long long)n_slots);
  for (int k = 0; k < K; ++k) {
    CHECK(sp.seg[k] >= kDkdvMinSeg, "segment of %d stages", sp.seg[k]);
    CHECK(sp.slot_off[k + 1] - sp.slot_off[k] <= kDkdvItemsTarget, "response %d has %d slots", k,
          sp.slot_off[k + 1] - sp.slot_off[k]);
  }
  // next stage expected per (k, gh, kt), and slot use
  std::vector<std::vector<int>> next(K);
  int64_t n_tiles = 0;
  for (int k = 0; k < K; ++k) {
    next[k].assign((size_t)Hkv * resp_tiles(g, k), 0);
    n_tiles += (int64_t)Hkv * resp_tiles(g, k);
  }
  CHECK(n_tiles == tiles, "tile count %lld vs %lld", (long long)n_tiles, (long long)tiles);
  std::vector<int> slot_used((size_t)n_slots, 0);
  for (int64_t idx = 0; idx < items + 8; ++idx) {
    const DkdvItem it = dkdv_item(g, pg, sp, (int)idx);
    if (idx >= items) {
      CHECK(it.k < 0, "item %lld past the end decodes to response %d", (long long)idx, it.k);
      continue;
    }
    if (it.k < 0 || it.k >= K || it.gh < 0 || it.gh >= Hkv || it.kt < 0 || it.kt >= resp_tiles(g, it.k)) {
      CHECK(false, "item %lld decodes to (%d, %d, %d)", (long long)idx, it.k, it.gh, it.kt);
      continue;
    }
    int& nx = next[it.k][(size_t)it.gh * resp_tiles(g, it.k) + it.kt];
    CHECK(it.t0 == nx, "item %lld starts at stage %d, expected %d", (long long)idx, it.t0, nx);
    CHECK(it.n_stages >= 1 && it.n_stages <= sp.seg[it.k], "item %lld has %d stages", (long long)idx, it.n_stages);
    nx = it.t0 + it.n_stages;
    const int n_seg = (pg.off[it.k + 1] - pg.off[it.k]) / kPgStageRows;
    const int j0 = it.kt * kRespKeys;
    const int s0 = ((j0 > row_lo ? j0 : row_lo) * g.grp - pg.m_lo) / kPgStageRows;
    const int lo_stage = it.n_top - it.n_stages, hi_stage = it.n_top - 1;
    CHECK(hi_stage < n_seg && lo_stage >= s0 && lo_stage >= 0, "item %lld stream stages [%d, %d] outside [%d, %d)",
          (long long)idx, lo_stage, hi_stage, s0, n_seg);
    if (it.seg_idx == 0) {
      CHECK(it.slot == -1, "first segment with slot %lld", (long long)it.slot);
    } else {
      const int64_t want = dkdv_tile_slot(g, pg, sp, it.k, it.gh, it.kt) + it.seg_idx - 1;
      CHECK(it.slot == want, "item %lld slot %lld, the reduction reads %lld", (long long)idx, (long long)it.slot,
            (long long)want);
      if (it.slot >= 0 && it.slot < n_slots) slot_used[(size_t)it.slot]++;
      else CHECK(false, "item %lld slot %lld outside [0, %lld)", (long long)idx, (long long)it.slot, (long long)n_slots);
    }
  }
  for (int k = 0; k < K; ++k)
    for (int gh = 0; gh < Hkv; ++gh)
      for (int kt = 0; kt < resp_tiles(g, k); ++kt)
        CHECK(next[k][(size_t)gh * resp_tiles(g, k) + kt] == resp_tile_stages(g, pg, k, kt),
              "tile (%d, %d, %d) covered up to stage %d of %d", k, gh, kt,
              next[k][(size_t)gh * resp_tiles(g, k) + kt], resp_tile_stages(g, pg, k, kt));
  for (int64_t i = 0; i < n_slots; ++i) CHECK(slot_used[(size_t)i] == 1, "slot %lld used %d times", (long long)i, slot_used[(size_t)i]);
}

// A call over K responses cuts each response's tiles exactly as a call of that response
// alone does (same segment length, same segments), so both sum every key's gradient in the
// same order.
static void check_dkdv_split_per_response(const std::vector<int>& lens, int R_max, int Hq, int Hkv) {
  auto plan = [&](const std::vector<int>& ls, int R) {
    rr_problem p{};
    p.P = 4096;
    p.chunk = 1024;
    p.R_max = R;
    p.K = (int)ls.size();
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.d_qk = p.d_v = 128;
    p.block = 2048;
    p.dtype = RR_BF16;
    p.tau = 0.088f;
    const Geom g = make_geom(&p, ls.data());
    const PgGeom pg = make_pg_geom(&p, ls.data(), 0, R);
    DkdvSplit sp{};
    int64_t n_slots = 0, tiles = 0;
    const int64_t items = plan_dkdv_split(g, pg, kDkdvItemsTarget, kDkdvMinSeg, sp, n_slots, tiles);
    // (k, gh, kt, seg_idx, t0, n_stages) of every item
    std::vector<std::vector<int>> out;
    for (int64_t i = 0; i < items; ++i) {
      const DkdvItem it = dkdv_item(g, pg, sp, (int)i);
      out.push_back({it.k, it.gh, it.kt, it.seg_idx, it.t0, it.n_stages});
    }
    return std::make_pair(sp, out);
  };
  const auto many = plan(lens, R_max);
  for (int k = 0; k < (int)lens.size(); ++k) {
    const auto one = plan({lens[k]}, lens[k] > 0 ? lens[k] : 1);
    CHECK(many.first.seg[k] == one.first.seg[0], "response %d: segment %d in the call, %d alone", k,
          many.first.seg[k], one.first.seg[0]);
    std::vector<std::vector<int>> mine;
    for (const auto& v : many.second)
      if (v[0] == k) mine.push_back({0, v[1], v[2], v[3], v[4], v[5]});
    CHECK(mine == one.second, "response %d is cut differently in the call of %zu", k, lens.size());
  }
}

static void check_dkdv_split() {
  check_dkdv_split_per_response({7666, 3930, 7116, 3152, 4233, 3153, 2159, 6650}, 8192, 24, 4);
  check_dkdv_split_per_response({520, 300, 65, 1}, 520, 24, 4);
  check_dkdv_split_per_response({90, 41, 7}, 96, 4, 1);
  // the 2M group's members one by one (24 query heads on 4 KV heads)
  for (int r : {7666, 3930, 7116, 3152, 4233, 3153, 2159, 6650}) check_dkdv_case(1, {r}, 8192, 24, 4, 0, 8192);
  check_dkdv_case(1, {4096}, 4096, 32, 8, 0, 4096);                 // GQA, 32 heads on 8
  check_dkdv_case(1, {8192}, 8192, 24, 4, 0, 8192);                 // one-rank share
  for (int b = 0; b < 4; ++b) check_dkdv_case(1, {8192}, 8192, 24, 4, 2048 * b, 2048 * (b + 1));   // block walk
  check_dkdv_case(1, {4096}, 4096, 32, 8, 2048, 4096);
  check_dkdv_case(8, {7666, 3930, 7116, 3152, 4233, 3153, 2159, 6650}, 8192, 24, 4, 0, 8192);   // one call
  check_dkdv_case(3, {1, 0, 300}, 384, 4, 1, 0, 384);               // tiny, empty and ragged
  check_dkdv_case(4, {256, 129, 128, 77}, 256, 4, 2, 0, 256);
  check_dkdv_case(2, {513, 1000}, 1000, 6, 2, 100, 700);           // a block walk with ragged ends
  check_dkdv_case(1, {0}, 64, 4, 1, 0, 64);                         // nothing to do
  std::printf("response dK/dV split: ok\n");
}

int main() {
  check_addresses();
  check_dkdv_split();
  check_pointers();
  check_accum();
  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("all host checks passed\n");
  return 0;
}
