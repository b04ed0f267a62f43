// Drives every entry point of the C ABI (api.cpp, built with the launcher
// stand-ins of launch_stubs.cpp) through valid and invalid arguments, under
// AddressSanitizer and UndefinedBehaviorSanitizer.  A valid call must return
// KVEVICT_OK and reach its launcher; an invalid one must return its error
// status and reach none.  The launchers themselves abort on sizes the
// validation should have rejected.  Prints "api ok" and exits 0 on success.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "kvevict.h"

extern int g_launches;

namespace {

int failures = 0;

void expect(kvevict_status got, kvevict_status want, int launches_before, bool launch,
            const char* what, int line) {
  const bool launched = g_launches > launches_before;
  if (got != want || launched != (launch && want == KVEVICT_OK)) {
    std::fprintf(stderr, "line %d (%s): status %d (want %d), launched %d\n", line, what, (int)got,
                 (int)want, (int)launched);
    ++failures;
  }
}

#define CHECK(call, want, launch)                                  \
  do {                                                             \
    const int before = g_launches;                                 \
    expect((call), (want), before, (launch), #call, __LINE__);     \
  } while (0)

// Non-null, 16-byte aligned addresses that the host code never dereferences.
template <typename T>
T* fake(uintptr_t k) {  // stand-in device addresses 1 TiB apart: the stores never overlap
  return reinterpret_cast<T*>(k << 40);
}

kvevict_kv_desc contig(int32_t D, int32_t H, int64_t cap) {
  return kvevict_kv_desc{KVEVICT_LAYOUT_CONTIG, D, H, 0, cap, cap * D, nullptr, 0};
}

kvevict_kv_desc paged(int32_t D, int32_t H, int32_t ps, int64_t pool, const int32_t* pt,
                      int64_t pt_ld) {
  return kvevict_kv_desc{KVEVICT_LAYOUT_PAGED, D, H, ps, pool, 0, pt, pt_ld};
}

}  // namespace

int main() {
  const kvevict_status OK = KVEVICT_OK, INV = KVEVICT_ERR_INVALID_ARG;
  const kvevict_status ALIGN = KVEVICT_ERR_ALIGNMENT, WS = KVEVICT_ERR_WORKSPACE;
  const kvevict_status UNSUP = KVEVICT_ERR_UNSUPPORTED;
  float* sc = fake<float>(1);
  int32_t* idx = fake<int32_t>(2);
  int32_t* cnt = fake<int32_t>(3);
  const int64_t big_req = (1LL << 32) - 1;
  const int32_t big = 2147483647;
  const int64_t huge = 1LL << 62;

  // random scores
  CHECK(kvevict_score_random(sc, 1088, 2, 3, 8, 1088, 128, 7, 0, 0, nullptr), OK, true);
  CHECK(kvevict_score_random(sc, 1088, 2, 3, 8, 1088, 128, 7, 0, 1, nullptr), OK, true);
  CHECK(kvevict_score_random(sc, 1087, 2, 3, 8, 1088, 128, 7, 0, 0, nullptr), INV, false);
  CHECK(kvevict_score_random(sc, 1088, 2, 3, 8, 1088, 1089, 7, 0, 0, nullptr), INV, false);
  CHECK(kvevict_score_random(nullptr, 1088, 2, 3, 8, 1088, 0, 7, 0, 0, nullptr), INV, false);
  CHECK(kvevict_score_random(sc, 16, big_req, big, big, 16, 0, 7, 0, 0, nullptr), INV, false);
  CHECK(kvevict_score_random(sc, 16, 1LL << 32, 1, 1, 16, 0, 7, 0, 0, nullptr), INV, false);

  // weighted scores
  const int32_t wb[2] = {0, 0}, wc[2] = {3, 6}, wc_bad[2] = {3, 7}, wb_bad[2] = {0, 1};
  const float* sig = fake<const float>(4);
  CHECK(kvevict_score_weighted(sc, 64, sig, sig, 64 * 8, 8, 1, sig, 6, wb, wc, 2, 4, 6, 8, 64, 4,
                               nullptr), OK, true);
  CHECK(kvevict_score_weighted(sc, 64, sig, sig, 64 * 8, 8, 1, sig, 6, wb, wc_bad, 2, 4, 6, 8, 64,
                               4, nullptr), INV, false);
  CHECK(kvevict_score_weighted(sc, 64, sig, sig, 64 * 8, 8, 1, sig, 6, wb_bad, wc, 2, 4, 6, 8, 64,
                               4, nullptr), INV, false);
  CHECK(kvevict_score_weighted(sc, 64, sig, sig, 64 * 8, 8, 1, sig, 6, nullptr, wc, 2, 4, 6, 8, 64,
                               4, nullptr), INV, false);
  CHECK(kvevict_score_weighted(sc, 64, sig, sig, -1, 8, 1, sig, 6, wb, wc, 2, 4, 6, 8, 64, 4,
                               nullptr), INV, false);

  // top-K and random draw + top-K
  CHECK(kvevict_select_topk(idx, 1024, sc, 1088, 10, 1088, 1024, 128, nullptr), OK, true);
  CHECK(kvevict_select_topk(idx, 1023, sc, 1088, 10, 1088, 1024, 128, nullptr), INV, false);
  CHECK(kvevict_select_topk(idx, 1024, sc, 1088, 10, 1088, 1024, 1025, nullptr), INV, false);
  CHECK(kvevict_select_topk(idx, 1024, sc, 1088, -1, 1088, 1024, 128, nullptr), INV, false);
  CHECK(kvevict_select_random(idx, 1024, 128, 36, 8, 1088, 1024, 128, 1, 2, 0, nullptr), OK, true);
  CHECK(kvevict_select_random(idx, 1024, big_req, big, big, 1088, 1024, 128, 1, 2, 0, nullptr),
        INV, false);
  CHECK(kvevict_select_random(idx, 1024, big_req, big, 8, 1088, 1024, 128, 1, 2, 1, nullptr), INV,
        false);

  // per-layer budgets: host arithmetic, checked for its totals
  for (int32_t L = 1; L <= 64; L += 7) {
    for (double p : {0.0, 0.1, 0.25, 0.5, 0.999, 1.0}) {
      std::vector<float> gate(L);
      for (int32_t l = 0; l < L; ++l) gate[l] = 0.022f + 0.437f * (float)((l * 37) % 64) / 63.0f;
      std::vector<int32_t> bud(L, -1);
      const int32_t n_body = 32512;
      CHECK(kvevict_layer_power_budget(gate.data(), L, n_body, p, bud.data()), OK, false);
      int64_t total = 0;
      for (int32_t l = 0; l < L; ++l) {
        if (bud[l] < 0 || bud[l] > n_body) ++failures;
        total += bud[l];
      }
      if (total != (int64_t)L * (int64_t)std::nearbyint(p * n_body)) {
        std::fprintf(stderr, "layer budget total %lld for L=%d p=%g\n", (long long)total, L, p);
        ++failures;
      }
    }
  }
  {
    const float g3[3] = {0.1f, NAN, 0.2f};
    int32_t b3[3];
    CHECK(kvevict_layer_power_budget(g3, 3, 100, 0.5, b3), INV, false);
    CHECK(kvevict_layer_power_budget(g3, 3, 100, 1.5, b3), INV, false);
  }
  const int32_t lb[4] = {100, 200, 300, 400}, lb_bad[4] = {100, 200, 300, 961};
  CHECK(kvevict_select_topk_layers(idx, 1088, cnt, sc, 1088, 8, 4, 8, 1088, 128, lb, nullptr), OK,
        true);
  CHECK(kvevict_select_topk_layers(idx, 1088, cnt, sc, 1088, 8, 4, 8, 1088, 128, lb_bad, nullptr),
        INV, false);
  CHECK(kvevict_select_topk_layers(idx, 1088, cnt, sc, 1088, 6, 4, 8, 1088, 128, lb, nullptr), INV,
        false);  // not whole requests
  CHECK(kvevict_select_topk_layers(idx, 1088, cnt, sc, 1088, huge, 4, 8, 1088, 128, lb, nullptr),
        INV, false);
  CHECK(kvevict_reduce_max_heads(sc, 1088, sc, 1088, 10, 8, 1088, nullptr), OK, true);
  CHECK(kvevict_reduce_max_heads(sc, 1087, sc, 1088, 10, 8, 1088, nullptr), INV, false);
  CHECK(kvevict_reduce_max_heads(sc, 1088, sc, 1088, huge, 8, 1088, nullptr), INV, false);

  // global top-B: workspace protocol
  size_t wsb = 0;
  int64_t budget = -1;
  CHECK(kvevict_select_global(idx, 32768, cnt, &budget, sc, 32768, 64, 32768, 256, 0.25, nullptr,
                              &wsb, nullptr), OK, false);
  std::vector<uint8_t> ws_host;  // only its address is used
  void* ws = fake<void>(5);
  size_t small = wsb - 1;
  CHECK(kvevict_select_global(idx, 32768, cnt, &budget, sc, 32768, 64, 32768, 256, 0.25, ws,
                              &small, nullptr), WS, false);
  CHECK(kvevict_select_global(idx, 32768, cnt, &budget, sc, 32768, 64, 32768, 256, 0.25, ws, &wsb,
                              nullptr), OK, true);
  if (budget != 64LL * 8128) {
    std::fprintf(stderr, "global budget %lld\n", (long long)budget);
    ++failures;
  }
  CHECK(kvevict_select_global(idx, 32768, cnt, &budget, sc, 32768, 64, 32768, 256, NAN, ws, &wsb,
                              nullptr), INV, false);
  CHECK(kvevict_select_global(idx, 32768, cnt, &budget, sc, 32768, huge, 32768, 256, 0.25, nullptr,
                              &wsb, nullptr), INV, false);
  CHECK(kvevict_select_global(idx, 32768, cnt, &budget, sc, 32768, 64, 32768, 256, 0.25, ws,
                              nullptr, nullptr), INV, false);
  CHECK(kvevict_select_global(idx, 32768, cnt, &budget, sc, 32768, 64, 32768, 256, 0.25,
                              fake<uint8_t>(5) + 2, &wsb, nullptr), ALIGN, false);
  // allocation-free variant: the static array's size bounds the call
  CHECK(kvevict_select_global_noalloc(idx, 32768, cnt, &budget, sc, 32768, 64, 32768, 256, 0.25,
                                      nullptr), OK, true);
  CHECK(kvevict_select_global_noalloc(idx, 100, cnt, &budget, sc, 100, 65600, 100, 10, 0.3,
                                      nullptr), WS, false);  // more than the array holds
  CHECK(kvevict_select_global_noalloc(idx, 32768, cnt, &budget, sc, 32768, 64, 32768, 256, NAN,
                                      nullptr), INV, false);
  CHECK(kvevict_select_global_noalloc(idx, 32768, cnt, &budget, nullptr, 32768, 64, 32768, 256,
                                      0.25, nullptr), INV, false);  // no scores
  size_t wsb2 = 0;
  CHECK(kvevict_score_select_global(idx, 32768, cnt, &budget, sc, 32768, sig, sig, 32768 * 48, 48,
                                    1, sig, 6, wb, wc, 2, 4, 6, 48, 32768, 256, 0.25, nullptr,
                                    &wsb2, nullptr), OK, false);
  CHECK(kvevict_score_select_global(idx, 32768, cnt, &budget, sc, 32768, sig, sig, 32768 * 48, 48,
                                    1, sig, 6, wb, wc, 2, 4, 6, 48, 32768, 256, 0.25, ws, &wsb2,
                                    nullptr), OK, true);

  // compaction, out of place
  kvevict_kv_desc src = contig(128, 8, 1088), dst = contig(128, 8, 1024);
  void* ks = fake<void>(6);
  void* vs = fake<void>(7);
  void* kd = fake<void>(8);
  void* vd = fake<void>(9);
  CHECK(kvevict_compact(&src, ks, vs, &dst, kd, vd, idx, 1024, nullptr, 1024, 16, 8, nullptr,
                        nullptr), OK, true);
  CHECK(kvevict_compact(&src, ks, vs, &dst, kd, vd, idx, 1024, cnt, 1024, 16, 1, nullptr, nullptr),
        OK, true);
  CHECK(kvevict_compact(&src, ks, vs, &dst, kd, vd, idx, 1025, nullptr, 1025, 16, 8, nullptr,
                        nullptr), INV, false);  // K > dst rows
  CHECK(kvevict_compact(&src, ks, vs, &dst, vs, vd, idx, 1024, nullptr, 1024, 16, 8, nullptr,
                        nullptr), INV, false);  // K dst aliases V src
  {  // partial overlaps, by the descriptors' extents (16 groups x 8 heads)
    const int64_t src_bytes = 128LL * 1088 * 128 * 2, dst_bytes = 128LL * 1024 * 128 * 2;
    uint8_t* k8 = fake<uint8_t>(6);
    uint8_t* v8 = fake<uint8_t>(7);
    uint8_t* d8 = fake<uint8_t>(8);
    CHECK(kvevict_compact(&src, ks, vs, &dst, k8 + 4096, vd, idx, 1024, nullptr, 1024, 16, 8,
                          nullptr, nullptr), INV, false);  // K dst starts inside K src
    CHECK(kvevict_compact(&src, ks, vs, &dst, k8 - dst_bytes + 16, vd, idx, 1024, nullptr, 1024,
                          16, 8, nullptr, nullptr), INV, false);  // K dst runs into K src
    CHECK(kvevict_compact(&src, ks, vs, &dst, k8 + src_bytes, vd, idx, 1024, nullptr, 1024, 16, 8,
                          nullptr, nullptr), OK, true);  // touching, not overlapping
    CHECK(kvevict_compact(&src, ks, vs, &dst, kd, v8 + src_bytes - 16, idx, 1024, nullptr, 1024,
                          16, 8, nullptr, nullptr), INV, false);  // V dst in V src's last row
    CHECK(kvevict_compact(&src, ks, vs, &dst, kd, kd, idx, 1024, nullptr, 1024, 16, 8, nullptr,
                          nullptr), INV, false);  // K dst and V dst alias
    CHECK(kvevict_compact(&src, ks, vs, &dst, kd, d8 + dst_bytes - 16, idx, 1024, nullptr, 1024,
                          16, 8, nullptr, nullptr), INV, false);  // V dst in K dst's last row
    CHECK(kvevict_compact(&src, ks, k8 + 4096, &dst, kd, vd, idx, 1024, nullptr, 1024, 16, 8,
                          nullptr, nullptr), OK, true);  // overlapping sources are only read
  }
  CHECK(kvevict_compact(&src, fake<uint8_t>(6) + 8, vs, &dst, kd, vd, idx, 1024, nullptr, 1024, 16,
                        8, nullptr, nullptr), ALIGN, false);
  CHECK(kvevict_compact(&src, ks, vs, &dst, kd, vd, idx, 1024, nullptr, 1024, huge, 8, nullptr,
                        nullptr), INV, false);
  kvevict_kv_desc wrap = kvevict_kv_desc{KVEVICT_LAYOUT_CONTIG, 128, 8, 0, 1LL << 60, 1 << 20,
                                         nullptr, 0};
  CHECK(kvevict_compact(&wrap, ks, vs, &dst, kd, vd, idx, 1024, nullptr, 1024, 1, 8, nullptr,
                        nullptr), INV, false);
  const int32_t* pt = fake<const int32_t>(10);
  kvevict_kv_desc ps = paged(128, 8, 16, 304128, pt, 132), pd = paged(128, 8, 16, 294912, pt, 128);
  CHECK(kvevict_compact(&ps, ks, vs, &pd, kd, vd, idx, 2048, nullptr, 2048, 2304, 8, nullptr,
                        nullptr), OK, true);
  kvevict_kv_desc p12 = paged(128, 8, 12, 100, pt, 10), pnull = paged(128, 8, 16, 100, nullptr, 10);
  CHECK(kvevict_compact(&p12, ks, vs, &dst, kd, vd, idx, 1024, nullptr, 1024, 4, 8, nullptr,
                        nullptr), UNSUP, false);
  CHECK(kvevict_compact(&pnull, ks, vs, &dst, kd, vd, idx, 1024, nullptr, 1024, 4, 8, nullptr,
                        nullptr), INV, false);

  // KeyDiff
  kvevict_kv_desc keys = contig(128, 8, 1088);
  CHECK(kvevict_score_keydiff(sc, 1088, &keys, ks, 16, 1088, 128, nullptr), OK, true);
  kvevict_kv_desc keys96 = contig(96, 8, 1088);
  CHECK(kvevict_score_keydiff(sc, 1088, &keys96, ks, 16, 1088, 128, nullptr), UNSUP, false);
  CHECK(kvevict_score_keydiff(sc, 1088, &keys, ks, huge, 1088, 128, nullptr), INV, false);

  // ordered compaction into a paged destination: workspace protocol and checks
  {
    kvevict_kv_desc ps2 = paged(128, 8, 16, 304128, pt, 132), pd2 = paged(128, 8, 16, 294912, pt, 128);
    size_t ob = 0;
    CHECK(kvevict_compact_ordered(&ps2, ks, vs, &pd2, kd, vd, idx, 2048, nullptr, 2048, 2304, 8,
                                  nullptr, nullptr, &ob, nullptr), OK, false);  // size query
    if (ob != (294912 * 4 + 256 + 255) / 256 * 256) {
      std::fprintf(stderr, "ordered workspace %zu\n", ob);
      ++failures;
    }
    void* ows = fake<void>(14);
    CHECK(kvevict_compact_ordered(&ps2, ks, vs, &pd2, kd, vd, idx, 2048, nullptr, 2048, 2304, 8,
                                  nullptr, ows, &ob, nullptr), OK, true);
    size_t small = ob - 1;
    CHECK(kvevict_compact_ordered(&ps2, ks, vs, &pd2, kd, vd, idx, 2048, nullptr, 2048, 2304, 8,
                                  nullptr, ows, &small, nullptr), WS, false);
    CHECK(kvevict_compact_ordered(&ps2, ks, vs, &pd2, kd, vd, idx, 2048, nullptr, 2048, 2304, 8,
                                  nullptr, fake<uint8_t>(8) + 4096, &ob, nullptr), INV, false);
    CHECK(kvevict_compact_ordered(&ps2, ks, vs, &pd2, kd, vd, idx, 2048, nullptr, 2048, 2304, 8,
                                  nullptr, fake<uint8_t>(14) + 64, &ob, nullptr), ALIGN, false);
  }

  // whole-page copies
  {
    const int32_t* ids = fake<const int32_t>(13);
    CHECK(kvevict_copy_pages(ks, vs, 304128, ids, kd, vd, 294912, ids, 294912, 32768, nullptr,
                             nullptr), OK, true);
    CHECK(kvevict_copy_pages(ks, vs, 304128, ids, kd, vd, 294912, ids, 0, 32768, nullptr,
                             nullptr), OK, false);  // nothing to copy
    CHECK(kvevict_copy_pages(ks, vs, 304128, ids, kd, vd, 294912, ids, 10, 24, nullptr, nullptr),
          ALIGN, false);
    CHECK(kvevict_copy_pages(ks, vs, 304128, ids, fake<uint8_t>(6) + 4096, vd, 294912, ids, 10,
                             32768, nullptr, nullptr), INV, false);  // K dst inside K src
    CHECK(kvevict_copy_pages(ks, vs, 304128, ids, kd, kd, 294912, ids, 10, 32768, nullptr,
                             nullptr), INV, false);  // the destinations alias
    CHECK(kvevict_copy_pages(ks, vs, 1LL << 62, ids, kd, vd, 294912, ids, 10, 1024, nullptr,
                             nullptr), INV, false);  // pool size overflows
    CHECK(kvevict_copy_pages(ks, vs, 30, ids, fake<uint8_t>(6) + 30 * 32768, vd, 30, ids, 10,
                             32768, nullptr, nullptr), OK, true);  // pools that touch
  }

  // in place
  uint32_t* fc = fake<uint32_t>(11);
  int32_t* fp = fake<int32_t>(12);
  kvevict_kv_desc store = contig(128, 8, 3136);
  CHECK(kvevict_compact_inplace(&store, ks, vs, idx, 3072, nullptr, 3072, 3136, 16, 8, nullptr,
                                nullptr, nullptr, nullptr), OK, true);
  CHECK(kvevict_compact_inplace(&store, ks, ks, idx, 3072, nullptr, 3072, 3136, 16, 8, nullptr,
                                nullptr, nullptr, nullptr), INV, false);  // K and V the same
  CHECK(kvevict_compact_inplace(&store, ks, fake<uint8_t>(6) + 128LL * 3136 * 128 * 2 - 16, idx,
                                3072, nullptr, 3072, 3136, 16, 8, nullptr, nullptr, nullptr,
                                nullptr), INV, false);  // V starts in K's last row
  CHECK(kvevict_compact_inplace(&store, ks, fake<uint8_t>(6) + 128LL * 3136 * 128 * 2, idx, 3072,
                                nullptr, 3072, 3136, 16, 8, nullptr, nullptr, nullptr, nullptr),
        OK, true);  // V begins where K ends
  CHECK(kvevict_compact_inplace(&store, ks, vs, idx, 3072, nullptr, 3072, 3136, huge, 8, nullptr,
                                nullptr, nullptr, nullptr), INV, false);
  kvevict_kv_desc pstore = paged(128, 8, 16, 304128, pt, 132);
  CHECK(kvevict_compact_inplace(&pstore, ks, vs, idx, 2048, nullptr, 2048, 2112, 2304, 8, fp, fc,
                                nullptr, nullptr), OK, true);
  CHECK(kvevict_compact_inplace(&pstore, ks, vs, idx, 2048, nullptr, 2048, 2112, 2304, 8, nullptr,
                                fc, nullptr, nullptr), INV, false);  // no free list
  CHECK(kvevict_evict_random_inplace(&pstore, ks, vs, 64, 36, 2112, 2048, 1024, 1, 2, 0, nullptr,
                                     0, fp, fc, nullptr, nullptr), OK, true);
  CHECK(kvevict_evict_random_inplace(&store, ks, vs, big_req, big, 3136, 3072, 557, 1, 2, 0,
                                     nullptr, 0, fp, fc, nullptr, nullptr), INV, false);
  kvevict_kv_desc long_store = contig(128, 8, 40000);
  CHECK(kvevict_evict_random_inplace(&long_store, ks, vs, 1, 1, 40000, 20000, 0, 1, 2, 0, nullptr,
                                     0, fp, fc, nullptr, nullptr), UNSUP, false);
  int32_t* tab = fake<int32_t>(13);
  CHECK(kvevict_evict_pages_random(tab, 132, 16, 64, 36, 2112, 2048, 1024, 1, 2, nullptr, 0, fp,
                                   fc, nullptr), OK, true);
  CHECK(kvevict_evict_pages_random(tab, 132, 16, 64, 36, 2112, 2040, 1024, 1, 2, nullptr, 0, fp,
                                   fc, nullptr), INV, false);  // K not whole pages
  CHECK(kvevict_evict_pages_random(tab, 131, 16, 64, 36, 2112, 2048, 1024, 1, 2, nullptr, 0, fp,
                                   fc, nullptr), INV, false);  // table row too short

  // strings and version
  for (int s = 0; s <= 6; ++s)
    if (!kvevict_status_string((kvevict_status)s)) ++failures;
  if (kvevict_abi_version() < 1) ++failures;

  if (failures) {
    std::fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  std::printf("api ok: %d launches\n", g_launches);
  return 0;
}
