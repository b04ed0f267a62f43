// Runs every function the CPU oracle exports on small inputs, edge cases
// included, under AddressSanitizer and UndefinedBehaviorSanitizer, and checks
// the invariants the pages fix: the prompt is kept, kept indices ascend
// strictly, |S| = K per head and the counts add up to L*H*prot + B globally,
// compacted rows equal their sources.  Prints "oracle ok" and exits 0.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <vector>

extern "C" {
void oracle_philox4x64_10(const uint64_t* ctr, const uint64_t* key, uint64_t* out);
float oracle_random_draw(uint64_t seed, uint64_t request, uint64_t layer, uint64_t head,
                         uint64_t round, int64_t i);
void oracle_score_random(float* scores, int64_t ld, int32_t L, int32_t H, int32_t n, int32_t prot,
                         uint64_t seed, uint32_t round, int32_t shared_draw, int64_t list_begin,
                         int64_t list_end);
void oracle_score_weighted(float* out, int64_t ld, const float* beta, const float* vnorm,
                           int64_t sg, int64_t st, int64_t sj, const float* w, int32_t w_slots,
                           const int32_t* win_begin, const int32_t* win_count, int32_t L,
                           int32_t H, int32_t Hg, int32_t n, int32_t prot, int32_t t_begin,
                           int32_t t_end);
void oracle_select_topk(int32_t* kept, int64_t kept_ld, const float* scores, int64_t ld,
                        int64_t num_lists, int32_t n, int32_t K, int32_t prot);
int64_t oracle_budget(int64_t num_lists, int32_t n, int32_t prot, double p);
int64_t oracle_select_global(int32_t* kept, int64_t kept_ld, int32_t* kept_count,
                             const float* scores, int64_t ld, int64_t num_lists, int32_t n,
                             int32_t prot, double p);
void oracle_compact(int32_t src_paged, const uint16_t* k_src, const uint16_t* v_src,
                    int64_t src_list_stride, const int32_t* src_pt, int64_t src_pt_ld,
                    int32_t dst_paged, uint16_t* k_dst, uint16_t* v_dst, int64_t dst_list_stride,
                    const int32_t* dst_pt, int64_t dst_pt_ld, int32_t D, int32_t H,
                    int32_t page_size, const int32_t* kept, int64_t kept_ld,
                    const int32_t* kept_count, int32_t K, int64_t group_begin, int64_t group_end,
                    int32_t ipg);
}

namespace {

int failures = 0;

void fail(const char* what, int a, int b) {
  std::fprintf(stderr, "%s (%d, %d)\n", what, a, b);
  ++failures;
}

// kept[0, count) holds [0, prot) and then strictly increasing indices < n
void check_keep_set(const int32_t* kept, int32_t count, int32_t prot, int32_t n) {
  for (int32_t j = 0; j < count; ++j) {
    if (j < prot && kept[j] != j) fail("prompt not kept", j, kept[j]);
    if (kept[j] < 0 || kept[j] >= n) fail("index out of range", j, kept[j]);
    if (j > 0 && kept[j] <= kept[j - 1]) fail("indices not increasing", j, kept[j]);
  }
}

}  // namespace

int main() {
  // generator: blocks differ with every counter word, draws lie in [0, 1)
  uint64_t ctr[4] = {0, 0, 0, 0}, key[2] = {0, 0}, a[4], b[4];
  oracle_philox4x64_10(ctr, key, a);
  ctr[3] = 1;
  oracle_philox4x64_10(ctr, key, b);
  if (std::memcmp(a, b, sizeof a) == 0) fail("philox ignores a counter word", 0, 0);
  for (int64_t i = 0; i < 1000; ++i) {
    const float u = oracle_random_draw(7, 3, 2, 1, 5, i);
    if (!(u >= 0.0f && u < 1.0f)) fail("draw outside [0, 1)", (int)i, 0);
  }

  // random scores, per-head and shared, then top-K over them
  for (int shared = 0; shared < 2; ++shared) {
    const int32_t L = 2, H = 3, n = 97, prot = 5;
    const int64_t lists = (int64_t)L * (shared ? 1 : H) * 2;  // two requests
    std::vector<float> s(lists * (n + 3), -7.0f);
    oracle_score_random(s.data(), n + 3, L, H, n, prot, 11, 4, shared, 0, lists);
    for (int64_t l = 0; l < lists; ++l)
      for (int32_t i = 0; i < prot; ++i)
        if (!std::isinf(s[l * (n + 3) + i])) fail("prompt score not +inf", (int)l, i);
    for (int32_t K : {prot, 40, n}) {
      std::vector<int32_t> kept(lists * (K + 2), -1);
      oracle_select_topk(kept.data(), K + 2, s.data(), n + 3, lists, n, K, prot);
      for (int64_t l = 0; l < lists; ++l) check_keep_set(&kept[l * (K + 2)], K, prot, n);
    }
  }

  // top-K with NaN, infinities, signed zeros and ties
  {
    const float nan = std::numeric_limits<float>::quiet_NaN();
    const float inf = std::numeric_limits<float>::infinity();
    const std::vector<float> s = {0.5f, nan, -0.0f, 0.0f, inf, -inf, 0.5f, 1.0f, nan, 0.25f};
    const int32_t n = (int32_t)s.size();
    for (int32_t K = 0; K <= n; ++K) {
      std::vector<int32_t> kept(K + 1, -1);
      oracle_select_topk(kept.data(), K + 1, s.data(), n, 1, n, K, 0);
      check_keep_set(kept.data(), K, 0, n);
    }
  }

  // weighted scores: windows of 0, 3 and 6 GDN layers, a token range
  {
    const int32_t G = 8, n = 40, Hg = 5, L = 3, H = 2, S = 6, prot = 3;
    std::vector<float> beta(G * n * Hg), vnorm(G * n * Hg), w(L * H * S * Hg);
    for (size_t i = 0; i < beta.size(); ++i) {
      beta[i] = 0.1f + 0.8f * (float)((i * 2654435761u) % 1000) / 1000.0f;
      vnorm[i] = 0.5f + (float)((i * 40503u) % 1000) / 500.0f;
    }
    for (size_t i = 0; i < w.size(); ++i) w[i] = (float)((int)(i % 7) - 3);
    const int32_t wb[3] = {0, 0, 2}, wc[3] = {0, 3, 6};
    std::vector<float> out(L * H * n, -1.0f);
    oracle_score_weighted(out.data(), n, beta.data(), vnorm.data(), (int64_t)n * Hg, Hg, 1,
                          w.data(), S, wb, wc, L, H, Hg, n, prot, 0, n);
    oracle_score_weighted(out.data(), n, beta.data(), vnorm.data(), (int64_t)n * Hg, Hg, 1,
                          w.data(), S, wb, wc, L, H, Hg, n, prot, 10, 20);
    for (int32_t h = 0; h < H; ++h)
      for (int32_t t = prot; t < n; ++t)
        if (out[(0 * H + h) * n + t] != 0.0f) fail("empty window scores nonzero", h, t);
  }

  // global top-B: counts add up to lists*prot + B for several p, ties included
  {
    const int32_t n = 53, prot = 4;
    const int64_t lists = 5;
    std::vector<float> s(lists * n);
    for (size_t i = 0; i < s.size(); ++i) s[i] = (float)((i * 7919u) % 13) / 13.0f;
    for (double p : {0.0, 0.1, 0.37, 0.5, 1.0}) {
      std::vector<int32_t> kept(lists * n, -1), cnt(lists, -1);
      const int64_t B = oracle_select_global(kept.data(), n, cnt.data(), s.data(), n, lists, n,
                                             prot, p);
      if (B != oracle_budget(lists, n, prot, p)) fail("budget differs", (int)B, 0);
      int64_t total = 0;
      for (int64_t l = 0; l < lists; ++l) {
        check_keep_set(&kept[l * n], cnt[l], prot, n);
        total += cnt[l];
      }
      if (total != lists * prot + B) fail("global counts do not add up", (int)total, (int)B);
    }
    std::vector<int32_t> kept(1, -1), cnt(1, -1);
    oracle_select_global(kept.data(), 1, cnt.data(), s.data(), 1, 1, 1, 1, 0.5);  // no candidates
    if (cnt[0] != 1) fail("prompt-only list", cnt[0], 0);
  }

  // compaction: contiguous to contiguous, per-head and shared index lists,
  // variable counts; paged to paged through permuted tables
  {
    const int32_t D = 16, H = 2, n = 48, K = 20, ps = 16;
    const int64_t groups = 3;
    std::vector<uint16_t> ks(groups * H * n * D), vs(ks.size());
    for (size_t i = 0; i < ks.size(); ++i) {
      ks[i] = (uint16_t)(i * 31u);
      vs[i] = (uint16_t)(i * 17u + 5u);
    }
    std::vector<int32_t> kept(groups * H * K);
    for (int64_t l = 0; l < groups * H; ++l)
      for (int32_t j = 0; j < K; ++j) kept[l * K + j] = 2 * j + (int32_t)(l % 2);
    std::vector<int32_t> cnt(groups * H);
    for (int64_t l = 0; l < groups * H; ++l) cnt[l] = (int32_t)(l * 3 % (K + 1));
    for (int ipg : {H, 1}) {
      for (int var = 0; var < 2; ++var) {
        std::vector<uint16_t> kd(groups * H * K * D, 0), vd(kd.size(), 0);
        oracle_compact(0, ks.data(), vs.data(), (int64_t)n * D, nullptr, 0, 0, kd.data(),
                       vd.data(), (int64_t)K * D, nullptr, 0, D, H, ps, kept.data(), K,
                       var ? cnt.data() : nullptr, K, 0, groups, ipg);
        for (int64_t g = 0; g < groups; ++g)
          for (int32_t h = 0; h < H; ++h) {
            const int64_t il = g * ipg + (ipg == 1 ? 0 : h), l = g * H + h;
            const int32_t c = var ? cnt[il] : K;
            for (int32_t j = 0; j < c; ++j)
              if (std::memcmp(&kd[(l * K + j) * D], &ks[(l * n + kept[il * K + j]) * D],
                              D * 2) != 0 ||
                  std::memcmp(&vd[(l * K + j) * D], &vs[(l * n + kept[il * K + j]) * D],
                              D * 2) != 0)
                fail("compacted row differs", (int)l, j);
          }
      }
    }
    // paged: pools of 16-token pages [page][16][H][D], tables permuted per group
    const int32_t P = n / ps, Pd = (K + ps - 1) / ps;
    std::vector<int32_t> spt(groups * P), dpt(groups * Pd);
    for (int64_t i = 0; i < groups * P; ++i) spt[i] = (int32_t)((i * 5 + 3) % (groups * P));
    for (int64_t i = 0; i < groups * Pd; ++i) dpt[i] = (int32_t)((i * 7 + 1) % (groups * Pd));
    std::vector<uint16_t> kpd(groups * Pd * ps * H * D, 0), vpd(kpd.size(), 0);
    oracle_compact(1, ks.data(), vs.data(), 0, spt.data(), P, 1, kpd.data(), vpd.data(), 0,
                   dpt.data(), Pd, D, H, ps, kept.data(), K, nullptr, K, 0, groups, H);
    for (int64_t g = 0; g < groups; ++g)
      for (int32_t h = 0; h < H; ++h)
        for (int32_t j = 0; j < K; ++j) {
          const int32_t t = kept[(g * H + h) * K + j];
          const int64_t srow = ((int64_t)spt[g * P + t / ps] * ps + t % ps) * H + h;
          const int64_t drow = ((int64_t)dpt[g * Pd + j / ps] * ps + j % ps) * H + h;
          if (std::memcmp(&kpd[drow * D], &ks[srow * D], D * 2) != 0)
            fail("paged row differs", (int)g, j);
        }
  }

  if (failures) {
    std::fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  std::printf("oracle ok\n");
  return 0;
}
