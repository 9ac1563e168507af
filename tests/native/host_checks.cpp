// Host-compiled checks of the library's integer and host logic (no GPU): the address
// arithmetic of the direct global->LDS loads (csrc/k_addr.h, the functions the kernels
// call), the classification of pointer lookups, and the accumulation window's
// version/resident checks (csrc/rr_validate.cpp).  Built and run by
// tests/test_host_native.py; prints one line per group and exits non-zero on the first
// failure.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "k_addr.h"
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

static void check_rows_shape(const RowsShape& sh, uint32_t stride) {
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
          CHECK((uint64_t)a.src_off + 16 <= (uint64_t)rows_valid * stride, "load past the stage's rows");
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

int main() {
  check_addresses();
  check_pointers();
  check_accum();
  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("all host checks passed\n");
  return 0;
}
