// Host-only checks of the TTT library, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (no GPU is needed or touched):
//
//  1. The stream-K split of the MFMA gradient kernel and the slot arithmetic
//     of its update kernel, exhaustively over many (pairs, tiles per pair,
//     grid) shapes, mirroring how the two kernels walk them: every (pair, tile)
//     is covered by exactly one workgroup, every partial slot a workgroup
//     writes is below G*J and is written once, each workgroup touches at most
//     J pairs, and the update kernel reads back exactly the slots that were
//     written for each pair, from workgroups q0..q1.  Integer work: bit-exact.
//     For the direct gradient step: a pair is held whole by one workgroup
//     (the kernel's own test: a segment from the pair's first to its last
//     tile) exactly when its first and last workgroups coincide (q0 == q1,
//     the test the update kernel and the host use to skip it), and with one
//     workgroup per pair (G = P) workgroup q's range is exactly pair q.
//     The stream-K update kernel's index maps (sk_part_elem: the gradient
//     kernel's register order of a partial; sk_update_block: the matrix block
//     a 256-float4 workgroup covers), for every hidden width: each float4's
//     four elements lie in its workgroup's block, land on distinct slots of
//     the block's LDS copy, the row-order read-back covers the block exactly,
//     and the partial covers every element of both matrices exactly once.
//  2. The C ABI's host-side validation and workspace planning: bad configs and
//     bad forward arguments are rejected with the right status before anything
//     is enqueued, workspace sizes are 256-byte multiples, path names resolve.
//
// Exit status 0 means every check passed; the first failure is printed.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "ttt.h"
#include "ttt_internal.h"

static int g_fail = 0;
#define CHECK(cond, ...)                                        \
  do {                                                          \
    if (!(cond)) {                                              \
      if (!g_fail) {                                            \
        std::fprintf(stderr, "FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond); \
        std::fprintf(stderr, __VA_ARGS__);                      \
        std::fprintf(stderr, "\n");                             \
      }                                                         \
      g_fail = 1;                                               \
      return;                                                   \
    }                                                           \
  } while (0)

// ---------------------------------------------------------------------------
// 1. stream-K cover
static long long g_configs = 0, g_tiles = 0;

static void check_streamk(long long P, int tpp, long long target) {
  using namespace ttt;
  int G = 0, J = 0;
  sk_geometry(P, tpp, target, &G, &J);
  CHECK(G >= 1 && G <= target && G <= P * tpp, "P=%lld tpp=%d target=%lld G=%d", P, tpp, target, G);
  CHECK(J >= 1, "J=%d", J);
  const long long C = P * (tpp + kSkAlpha);
  std::vector<int> covered((size_t)(P * tpp), 0);
  std::vector<long long> slot_pair((size_t)G * J, -1);   // pair whose partial a slot holds
  std::vector<char> whole((size_t)P, 0);                 // some workgroup holds the pair entirely
  long long prev_end = 0;
  for (long long q = 0; q < G; ++q) {
    // as the gradient kernel: its tile range and segments
    const long long begin = sk_tile_at(q * C / G, tpp);
    const long long end = sk_tile_at((q + 1) * C / G, tpp);
    CHECK(begin == prev_end, "q=%lld begin %lld != previous end %lld (P=%lld tpp=%d G=%d)", q, begin, prev_end, P, tpp, G);
    CHECK(begin <= end, "q=%lld begin %lld > end %lld", q, begin, end);
    prev_end = end;
    const long long p_first = sk_first_pair(q, G, C, tpp);
    long long x = begin, pairs = 0;
    while (x < end) {
      const long long p = x / tpp;
      const long long seg_end = end < (p + 1) * tpp ? end : (p + 1) * tpp;
      const long long j = p - p_first;
      CHECK(j >= 0 && j < J, "q=%lld pair %lld slot offset %lld outside [0, J=%d) (P=%lld tpp=%d G=%d)", q, p, j, J, P,
            tpp, G);
      const long long slot = q * J + j;
      CHECK(slot < (long long)G * J, "slot %lld >= G*J", slot);
      CHECK(slot_pair[(size_t)slot] == -1, "slot %lld written twice", slot);
      slot_pair[(size_t)slot] = p;
      for (long long t = x; t < seg_end; ++t) covered[(size_t)t]++;
      if (x == p * tpp && seg_end == (p + 1) * tpp) whole[(size_t)p] = 1;
      ++pairs;
      x = seg_end;
    }
    CHECK(pairs <= J, "q=%lld touches %lld pairs > J=%d", q, pairs, J);
  }
  CHECK(prev_end == P * tpp, "last range ends at %lld, not %lld", prev_end, P * tpp);
  for (long long t = 0; t < P * tpp; ++t)
    CHECK(covered[(size_t)t] == 1, "tile %lld (pair %lld) covered %d times (P=%lld tpp=%d G=%d)", t, t / tpp,
          covered[(size_t)t], P, tpp, G);
  // as the update kernel: the slots it sums for each pair
  std::vector<int> read((size_t)G * J, 0);
  for (long long p = 0; p < P; ++p) {
    long long q0, q1;
    sk_pair_groups(p, tpp, G, C, &q0, &q1);
    CHECK(0 <= q0 && q0 <= q1 && q1 < G, "pair %lld groups [%lld, %lld]", p, q0, q1);
    CHECK((q0 == q1) == (whole[(size_t)p] != 0), "pair %lld: q0 %lld q1 %lld but held whole: %d (P=%lld tpp=%d G=%d)",
          p, q0, q1, (int)whole[(size_t)p], P, tpp, G);
    for (long long q = q0; q <= q1; ++q) {
      const long long s = sk_slot(p, q, q0, G, C, tpp, J);
      CHECK(s >= 0 && s < (long long)G * J, "pair %lld q %lld slot %lld out of range", p, q, s);
      CHECK(slot_pair[(size_t)s] == p, "pair %lld reads slot %lld of q=%lld, which holds pair %lld (P=%lld tpp=%d G=%d)",
            p, s, q, slot_pair[(size_t)s], P, tpp, G);
      read[(size_t)s]++;
    }
  }
  for (long long s = 0; s < (long long)G * J; ++s)
    CHECK((slot_pair[(size_t)s] >= 0) == (read[(size_t)s] == 1),
          "slot %lld written for pair %lld but read %d times", s, slot_pair[(size_t)s], read[(size_t)s]);
  ++g_configs;
  g_tiles += P * tpp;
}

// one workgroup per pair (the direct step's one-round grid, G = P, J = 1)
static void check_one_round(long long P, int tpp) {
  using namespace ttt;
  const long long G = P, C = P * (tpp + kSkAlpha);
  for (long long q = 0; q < G; ++q) {
    const long long begin = sk_tile_at(q * C / G, tpp), end = sk_tile_at((q + 1) * C / G, tpp);
    CHECK(begin == q * tpp && end == (q + 1) * tpp, "one round: q=%lld range [%lld, %lld) (P=%lld tpp=%d)", q, begin,
          end, P, tpp);
    CHECK(sk_first_pair(q, G, C, tpp) == q, "one round: q=%lld first pair %lld", q, sk_first_pair(q, G, C, tpp));
  }
}

static void streamk_sweep() {
  for (long long P = 1; P <= 1100; P += (P < 40 ? 1 : 37))
    for (int tpp = 1; tpp <= 600; tpp += (tpp < 12 ? 1 : tpp / 3)) { check_one_round(P, tpp); if (g_fail) return; }
  // the benchmarked shapes (ViT-S 384 pairs x 7 tiles, 1248^2 96 x 191, DiT
  // 48 x 512) at one and two workgroups per CU, then a dense sweep
  const long long targets[] = {1, 2, 3, 7, 64, 255, 256, 512, 1024};
  const long long real[][2] = {{384, 7}, {96, 191}, {48, 512}, {4, 64}, {6, 11}};
  for (auto& r : real)
    for (long long t : targets) { check_streamk(r[0], (int)r[1], t); if (g_fail) return; }
  for (long long P = 1; P <= 97; P += (P < 16 ? 1 : 9))
    for (int tpp = 1; tpp <= 400; tpp += (tpp < 12 ? 1 : tpp / 3))
      for (long long t : targets) { check_streamk(P, tpp, t); if (g_fail) return; }
}

// the stream-K update's block map, mirroring k_update_streamk: the LDS copy of
// a block has rows of cols + 4 floats; thread t reads float4 (t / (cols/4),
// 4 (t % (cols/4))) of it
static void check_update_blocks() {
  const int D = 64;
  for (int hid : {64, 128, 256}) {
    const int nf4 = D * hid / 2;                      // float4s of a pair's partial (both matrices)
    std::vector<int> seen(2 * D * hid, 0);
    for (int x = 0; x < nf4 / 256; ++x) {
      const ttt::SkBlock bk = ttt::sk_update_block(hid, x);
      CHECK(bk.rows * bk.cols == 1024, "hid %d x %d: block %d x %d", hid, x, bk.rows, bk.cols);
      CHECK(bk.cols % 4 == 0 && bk.col0 % 4 == 0 && bk.rs % 4 == 0, "hid %d x %d: float4 alignment", hid, x);
      const int ld = bk.cols + 4;
      std::vector<int> slot(bk.rows * ld, -1);       // LDS slot -> matrix element
      for (int t = 0; t < 256; ++t) {
        const int j = 256 * x + t;
        const ttt::SkElem el = ttt::sk_part_elem(hid, j);
        CHECK(el.mat == bk.mat, "hid %d j %d: matrix %d, block matrix %d", hid, j, el.mat, bk.mat);
        const int lr = el.row - bk.row0, lc = el.col - bk.col0;
        CHECK(lr >= 0 && lr + 3 < bk.rows && lc >= 0 && lc < bk.cols, "hid %d j %d: (%d, %d) outside the block", hid,
              j, el.row, el.col);
        for (int i = 0; i < 4; ++i) {
          const int s_ = (lr + i) * ld + lc;
          CHECK(slot[s_] == -1, "hid %d j %d: LDS slot %d written twice", hid, j, s_);
          const int e = (el.row + i) * bk.rs + el.col;
          slot[s_] = e;
          const int g = bk.mat * D * hid + e;
          CHECK(e >= 0 && e < D * hid && seen[g] == 0, "hid %d j %d: element %d out of range or repeated", hid, j, e);
          seen[g] = 1;
        }
      }
      for (int t = 0; t < 256; ++t) {                 // row-order read-back
        const int lr = t / (bk.cols / 4), lc = 4 * (t % (bk.cols / 4));
        const int e = (bk.row0 + lr) * bk.rs + bk.col0 + lc;
        for (int i = 0; i < 4; ++i)
          CHECK(slot[lr * ld + lc + i] == e + i, "hid %d x %d t %d: read-back of slot %d", hid, x, t, lr * ld + lc + i);
      }
    }
    for (int g = 0; g < 2 * D * hid; ++g) CHECK(seen[g] == 1, "hid %d: element %d of the pair not covered", hid, g);
  }
}

// ---------------------------------------------------------------------------
// 2. ABI host-side validation
static ttt_config cfg(int B = 2, int H = 3, int N = 100, int d = 64, int hidden = 256) {
  ttt_config c;
  std::memset(&c, 0, sizeof c);
  c.B = B; c.H = H; c.N = N; c.d = d; c.hidden = hidden;
  c.dtype = TTT_BF16; c.key_norm = 1; c.eps = 1e-5f; c.renorm = 0; c.flags = 0;
  return c;
}

static void abi_checks() {
  CHECK(ttt_version() == TTT_ABI_VERSION, "version");
  ttt_handle* h = nullptr;
  CHECK(ttt_create(nullptr, &h) == TTT_ERR_INVALID && h == nullptr, "NULL cfg");
  ttt_config c = cfg();
  CHECK(ttt_create(&c, nullptr) == TTT_ERR_INVALID, "NULL out");
  struct Bad { ttt_config c; int code; } bad[] = {
      {cfg(0), TTT_ERR_INVALID}, {cfg(1, 1, 0), TTT_ERR_INVALID}, {cfg(1, 1, 10, 129), TTT_ERR_UNSUPPORTED},
      {cfg(1, 1, 10, 0), TTT_ERR_UNSUPPORTED}, {cfg(1, 1, 10, 64, -1), TTT_ERR_INVALID}};
  for (auto& b : bad) {
    h = reinterpret_cast<ttt_handle*>(1);
    CHECK(ttt_create(&b.c, &h) == b.code && h == nullptr, "bad config not rejected (code %d)", b.code);
    CHECK(std::strlen(ttt_last_error(nullptr)) > 0, "no create error message");
  }
  c = cfg(); c.dtype = 7;
  CHECK(ttt_create(&c, &h) == TTT_ERR_INVALID, "dtype");
  c = cfg(); c.eps = std::nanf("");
  CHECK(ttt_create(&c, &h) == TTT_ERR_INVALID, "eps nan");
  c = cfg(); c.flags = 0x1000;
  CHECK(ttt_create(&c, &h) == TTT_ERR_INVALID, "flags");

  // workspace sizes and path names over the inner x loss x chunk x shape grid
  const int shapes[][5] = {{2, 3, 100, 64, 256}, {8, 12, 6084, 64, 256}, {2, 24, 16384, 64, 64}, {1, 4, 32768, 128, 256},
                           {1, 1, 1, 16, 48}, {64, 6, 196, 64, 64}, {3, 5, 77, 32, 512}};
  for (auto& s : shapes)
    for (int kn = 0; kn < 2; ++kn)
      for (int dt = 0; dt < 2; ++dt) {
        c = cfg(s[0], s[1], s[2], s[3], s[4]);
        c.key_norm = kn; c.dtype = dt;
        CHECK(ttt_create(&c, &h) == TTT_OK, "create %s", ttt_last_error(nullptr));
        for (int inner = 0; inner < 3; ++inner)
          for (int loss = 0; loss < 2; ++loss)
            for (int chunk : {0, 1, 64, 2048, 1 << 20}) {
              size_t n = 0;
              const int rc = ttt_workspace_bytes(h, loss, inner, chunk, &n);
              if (kn && chunk > 0) {
                CHECK(rc == TTT_ERR_UNSUPPORTED, "key norm + chunks accepted");
                CHECK(ttt_path_name(h, loss, inner, chunk) == nullptr, "path of a rejected request");
                continue;
              }
              if (chunk == 1 && s[2] > 65535) { CHECK(rc == TTT_ERR_UNSUPPORTED, "chunk count"); continue; }
              CHECK(rc == TTT_OK, "workspace_bytes: %s", ttt_last_error(h));
              CHECK(n > 0 && n % 256 == 0, "workspace %zu", n);
              CHECK(ttt_path_name(h, loss, inner, chunk) != nullptr, "path name");
            }
        size_t n = 0;
        CHECK(ttt_workspace_bytes(h, 9, 1, 0, &n) == TTT_ERR_INVALID, "bad loss");
        CHECK(ttt_workspace_bytes(h, 0, 9, 0, &n) == TTT_ERR_INVALID, "bad inner");
        CHECK(ttt_workspace_bytes(h, 0, 1, -1, &n) == TTT_ERR_INVALID, "bad chunk");
        CHECK(ttt_workspace_bytes(h, 0, 1, 0, nullptr) == TTT_ERR_INVALID, "NULL bytes");
        ttt_destroy(h);
      }

  // forward: every argument error is reported before anything is enqueued
  c = cfg();
  CHECK(ttt_create(&c, &h) == TTT_OK, "create");
  void* fake = reinterpret_cast<void*>(uintptr_t(1) << 20);   // never dereferenced
  ttt_weights W;
  std::memset(&W, 0, sizeof W);
  ttt_eta e = {1.0f, nullptr};
  CHECK(ttt_forward(h, nullptr, fake, fake, &W, &e, 0, 1, 0, fake, nullptr, fake, 1u << 30, nullptr) == TTT_ERR_INVALID,
        "NULL q");
  CHECK(ttt_forward(h, fake, fake, fake, &W, &e, 0, 1, 0, fake, nullptr, fake, 1u << 30, nullptr) == TTT_ERR_INVALID,
        "NULL W0");
  CHECK(ttt_forward(h, fake, fake, fake, nullptr, &e, 0, 1, 0, fake, nullptr, fake, 1u << 30, nullptr) == TTT_ERR_INVALID,
        "NULL W0 struct");
  W.w[0] = W.w[1] = static_cast<const float*>(fake);
  CHECK(ttt_forward(h, fake, fake, fake, &W, nullptr, 0, 1, 0, fake, nullptr, fake, 1u << 30, nullptr) == TTT_ERR_INVALID,
        "NULL eta");
  CHECK(ttt_forward(h, fake, fake, fake, &W, &e, 0, 1, 0, fake, nullptr, nullptr, 0, nullptr) == TTT_ERR_WORKSPACE,
        "NULL workspace");
  CHECK(ttt_forward(h, fake, fake, fake, &W, &e, 0, 1, 0, fake, nullptr, fake, 16, nullptr) == TTT_ERR_WORKSPACE,
        "small workspace");
  CHECK(ttt_forward(h, fake, fake, fake, &W, &e, 0, 1, 0, fake, nullptr, (char*)fake + 4, 1u << 30, nullptr) ==
            TTT_ERR_INVALID, "misaligned workspace");
  ttt_eta einf = {INFINITY, nullptr};
  CHECK(ttt_forward(h, fake, fake, fake, &W, &einf, 0, 1, 0, fake, nullptr, fake, 1u << 30, nullptr) == TTT_ERR_INVALID,
        "inf eta");
  W.batch_stride = 5;
  CHECK(ttt_forward(h, fake, fake, fake, &W, &e, 0, 1, 0, fake, nullptr, fake, 1u << 30, nullptr) == TTT_ERR_INVALID,
        "batch stride");
  CHECK(std::strstr(ttt_last_error(h), "batch_stride") != nullptr, "message");
  W.batch_stride = 0;
  CHECK(ttt_forward(h, fake, fake, fake, &W, &e, 0, 1, 16, fake, nullptr, fake, 1u << 30, nullptr) ==
            TTT_ERR_UNSUPPORTED, "key norm with chunks");
  CHECK(ttt_set_timing_events(h, nullptr, 3) == TTT_OK, "events off");
  void* evs[3] = {nullptr, nullptr, nullptr};
  CHECK(ttt_set_timing_events(h, evs, 3) == TTT_ERR_INVALID, "event count");
  CHECK(ttt_forward(nullptr, fake, fake, fake, &W, &e, 0, 1, 0, fake, nullptr, fake, 1u << 30, nullptr) ==
            TTT_ERR_INVALID, "NULL handle");
  CHECK(std::strcmp(ttt_status_string(TTT_OK), "ok") == 0, "status string");
  CHECK(std::strlen(ttt_status_string(12345)) > 0, "unknown status string");
  ttt_destroy(h);
  CHECK(ttt_destroy(nullptr) == TTT_OK, "destroy NULL");
}

int main() {
  streamk_sweep();
  if (!g_fail) std::printf("stream-K: %lld shapes, %lld tiles checked\n", g_configs, g_tiles);
  if (!g_fail) check_update_blocks();
  if (!g_fail) std::printf("stream-K update blocks checked\n");
  if (!g_fail) abi_checks();
  if (!g_fail) std::printf("ABI host checks passed\n");
  return g_fail;
}
