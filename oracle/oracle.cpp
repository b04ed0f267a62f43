// CPU oracle for the KV-cache eviction round.
//
// TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call
// this file: only the tests, the smoke check and the CPU-baseline leg of the
// benchmark use it. It shares no header, helper, constant table or kernel with
// the HIP library; it is written from the definitions on the pages:
//
//   * "Random Attention" blog summary (sungsoo.github.io, 2026-09-05),
//     Algorithm 1: draw a random score per entry, pin the prompt to +inf,
//     keep the top-K per KV head, return the keep set; the engine compacts the
//     kept entries per KV head in chronological order.  Shared draw: one keep
//     set for all heads.
//   * "GateSight" (signal-papers 2610.14754), problem statement: model-wide
//     budget B = 16*4*round(p*(n-prot)) exclusive of the protected prefix,
//     kept sets drawn from the non-prompt positions; the KVzip baseline ranks
//     (layer, head, token) scores globally (Sec. 5.1 baselines paragraph).
//     Sec. 4.1: the signals of the up to six GDN layers preceding an attention
//     layer (three for the first one); "log effective write" log(beta*|v|).
//
// Where the pages leave a step open the plainest reading is taken:
//   * rand: Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
//     numbers: as easy as 1, 2, 3", SC 2011), key (seed, 0), counter
//     (i/4, head, layer, request*2^32 + round), word i%4, top 24 bits -> [0,1).
//   * ties: the lower position (global: the lower flat index list*n+i) wins.
//   * NaN scores rank as -inf; -0 equals +0.
//   * round(): binary64 product, round half to even.
//   * weighted score: sum over window slots and GDN heads of
//     w * ln(beta * |v|), accumulated in binary64, rounded once to fp32.
//
// Everything here is deliberately plain: full stable sorts, one memcpy per row.

#include <algorithm>
#include <cfenv>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

namespace {

// ---------------------------------------------------------------------------
// Philox4x64-10 (Salmon et al., SC 2011, Sec. 4 and Table 2).
// One round: two 64x64->128 products of counter words 0 and 2 with the
// round multipliers; the new counter is (hi1^c1^k0, lo1, hi0^c3^k1, lo0).
// The key is bumped by the Weyl constants between rounds.
// ---------------------------------------------------------------------------
const uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ull;
const uint64_t kPhiloxM1 = 0xCA5A826395121157ull;
const uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ull;  // golden ratio
const uint64_t kPhiloxW1 = 0xBB67AE8584CAA73Bull;  // sqrt(3) - 1

void mul128(uint64_t a, uint64_t b, uint64_t* hi, uint64_t* lo) {
  unsigned __int128 p = (unsigned __int128)a * (unsigned __int128)b;
  *hi = (uint64_t)(p >> 64);
  *lo = (uint64_t)p;
}

void philox4x64_10(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4]) {
  uint64_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
  uint64_t k[2] = {key_in[0], key_in[1]};
  for (int round = 0; round < 10; ++round) {
    uint64_t hi0, lo0, hi1, lo1;
    mul128(kPhiloxM0, c[0], &hi0, &lo0);
    mul128(kPhiloxM1, c[2], &hi1, &lo1);
    uint64_t n0 = hi1 ^ c[1] ^ k[0];
    uint64_t n1 = lo1;
    uint64_t n2 = hi0 ^ c[3] ^ k[1];
    uint64_t n3 = lo0;
    c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
    k[0] += kPhiloxW0;
    k[1] += kPhiloxW1;
  }
  for (int w = 0; w < 4; ++w) out[w] = c[w];
}

// Random Attention score of slot i of the list (request, layer, head) in a
// given eviction round: 24 random bits scaled to [0, 1).  Exact in fp32.
float random_draw(uint64_t seed, uint64_t request, uint64_t layer, uint64_t head,
                  uint64_t round, int64_t i) {
  uint64_t ctr[4] = {(uint64_t)i / 4u, head, layer, (request << 32) | (round & 0xffffffffull)};
  uint64_t key[2] = {seed, 0};
  uint64_t out[4];
  philox4x64_10(ctr, key, out);
  uint64_t word = out[(uint64_t)i % 4u];
  double u = (double)(word >> 40) / 16777216.0;  // 2^24
  return (float)u;
}

// The ranking value of a score: NaN ranks below everything.
double rank_value(float s) {
  if (std::isnan(s)) return -std::numeric_limits<double>::infinity();
  return (double)s;  // -0 and +0 compare equal
}

}  // namespace

extern "C" {

// --- raw generator, exported for the known-answer tests --------------------
void oracle_philox4x64_10(const uint64_t* ctr, const uint64_t* key, uint64_t* out) {
  philox4x64_10(ctr, key, out);
}

float oracle_random_draw(uint64_t seed, uint64_t request, uint64_t layer, uint64_t head,
                         uint64_t round, int64_t i) {
  return random_draw(seed, request, layer, head, round, i);
}

// --- A2: Random Attention scores --------------------------------------------
// Lists are numbered list = (request*L + layer)*H + head (per-head draw) or
// list = request*L + layer (shared draw, one draw per layer from head 0).
// Writes scores[(list - list_begin)*ld + i] for lists in [list_begin, list_end).
// Slots i < prot are pinned to +inf (Algorithm 1, "prompt = +inf").
void oracle_score_random(float* scores, int64_t ld, int32_t L, int32_t H, int32_t n, int32_t prot,
                         uint64_t seed, uint32_t round, int32_t shared_draw,
                         int64_t list_begin, int64_t list_end) {
  const float inf = std::numeric_limits<float>::infinity();
  for (int64_t list = list_begin; list < list_end; ++list) {
    int64_t request, layer, head;
    if (shared_draw) {
      request = list / L;
      layer = list % L;
      head = 0;
    } else {
      request = list / ((int64_t)L * H);
      layer = (list / H) % L;
      head = list % H;
    }
    float* row = scores + (list - list_begin) * ld;
    for (int32_t i = 0; i < n; ++i) {
      row[i] = (i < prot) ? inf
                          : random_draw(seed, (uint64_t)request, (uint64_t)layer, (uint64_t)head,
                                        (uint64_t)round, i);
    }
  }
}

// --- A3: weighted GDN-signal scores ----------------------------------------
// s[l][h][t] = sum_{slot < win_count[l]} sum_{j < Hg}
//                 w[l][h][slot][j] * ln(beta[g][t][j] * vnorm[g][t][j]),
//              g = win_begin[l] + slot,
// for t >= prot; +inf for t < prot.  Signal element (g, t, j) sits at
// g*sg + t*st + j*sj.  Weights are [L][H][w_slots][Hg].  The product of two
// fp32 values is exact in binary64; the sum is accumulated in binary64 in the
// order written and rounded once to fp32.  Output row l*H + h, tokens
// [t_begin, t_end) written at out[(l*H+h)*ld + t].
void oracle_score_weighted(float* out, int64_t ld, const float* beta, const float* vnorm,
                           int64_t sg, int64_t st, int64_t sj, const float* w, int32_t w_slots,
                           const int32_t* win_begin, const int32_t* win_count, int32_t L,
                           int32_t H, int32_t Hg, int32_t n, int32_t prot, int32_t t_begin,
                           int32_t t_end) {
  const float inf = std::numeric_limits<float>::infinity();
  for (int32_t l = 0; l < L; ++l) {
    for (int32_t h = 0; h < H; ++h) {
      float* row = out + ((int64_t)l * H + h) * ld;
      for (int32_t t = t_begin; t < t_end && t < n; ++t) {
        if (t < prot) {
          row[t] = inf;
          continue;
        }
        double s = 0.0;
        for (int32_t slot = 0; slot < win_count[l]; ++slot) {
          int64_t g = (int64_t)win_begin[l] + slot;
          const float* wrow = w + (((int64_t)l * H + h) * w_slots + slot) * Hg;
          for (int32_t j = 0; j < Hg; ++j) {
            int64_t e = g * sg + (int64_t)t * st + (int64_t)j * sj;
            double x = std::log((double)beta[e] * (double)vnorm[e]);
            s += (double)wrow[j] * x;
          }
        }
        row[t] = (float)s;
      }
    }
  }
}

// --- A4: pin + per-head top-K ------------------------------------------------
// For each list: keep [0, prot), plus the K - prot best of [prot, n) ranked by
// score descending with the lower position first among equal scores (a stable
// sort of ascending positions).  kept[list*kept_ld + j], j < K, ascending.
void oracle_select_topk(int32_t* kept, int64_t kept_ld, const float* scores, int64_t ld,
                        int64_t num_lists, int32_t n, int32_t K, int32_t prot) {
  std::vector<int32_t> pos;
  for (int64_t list = 0; list < num_lists; ++list) {
    const float* s = scores + list * ld;
    pos.clear();
    for (int32_t i = prot; i < n; ++i) pos.push_back(i);
    std::stable_sort(pos.begin(), pos.end(),
                     [&](int32_t a, int32_t b) { return rank_value(s[a]) > rank_value(s[b]); });
    std::vector<int32_t> keep;
    for (int32_t i = 0; i < prot; ++i) keep.push_back(i);
    for (int32_t j = 0; j < K - prot; ++j) keep.push_back(pos[j]);
    std::sort(keep.begin(), keep.end());
    for (int32_t j = 0; j < K; ++j) kept[list * kept_ld + j] = keep[j];
  }
}

// --- model-wide budget ---------------------------------------------------------
// B = num_lists * round(p * (n - prot)), binary64 product, ties to even.
int64_t oracle_budget(int64_t num_lists, int32_t n, int32_t prot, double p) {
  std::fesetround(FE_TONEAREST);
  double per_list = std::nearbyint(p * (double)(n - prot));
  return num_lists * (int64_t)per_list;
}

// --- A5: pin + global top-B ----------------------------------------------------
// Keeps [0, prot) of every list plus the B best non-prompt entries over all
// lists, ranked by score descending with the lower flat index list*n + i first
// among equal scores.  Writes kept_count[list] and the ascending kept indices
// kept[list*kept_ld + j], j < kept_count[list].  Returns B.
int64_t oracle_select_global(int32_t* kept, int64_t kept_ld, int32_t* kept_count,
                             const float* scores, int64_t ld, int64_t num_lists, int32_t n,
                             int32_t prot, double p) {
  int64_t B = oracle_budget(num_lists, n, prot, p);
  std::vector<int64_t> flat;  // flat index list*n + i, in ascending order
  for (int64_t list = 0; list < num_lists; ++list)
    for (int32_t i = prot; i < n; ++i) flat.push_back(list * n + i);
  auto score_of = [&](int64_t f) { return rank_value(scores[(f / n) * ld + (f % n)]); };
  std::stable_sort(flat.begin(), flat.end(),
                   [&](int64_t a, int64_t b) { return score_of(a) > score_of(b); });
  int64_t take = std::min<int64_t>(B, (int64_t)flat.size());
  std::vector<std::vector<int32_t>> keep(num_lists);
  for (int64_t list = 0; list < num_lists; ++list)
    for (int32_t i = 0; i < prot; ++i) keep[list].push_back(i);
  for (int64_t r = 0; r < take; ++r) keep[flat[r] / n].push_back((int32_t)(flat[r] % n));
  for (int64_t list = 0; list < num_lists; ++list) {
    std::sort(keep[list].begin(), keep[list].end());
    kept_count[list] = (int32_t)keep[list].size();
    for (size_t j = 0; j < keep[list].size(); ++j) kept[list * kept_ld + j] = keep[list][j];
  }
  return B;
}

// --- A6: chronological compaction ------------------------------------------------
// A store holds bf16 rows of D elements (2*D bytes, copied verbatim).
//   contiguous: row (list, t) at element list*list_stride + t*D, where
//               list = group*H + head;
//   paged:      row (group, t, head) at element
//               ((page_table[group*pt_ld + t/page_size]*page_size + t%page_size)*H + head)*D.
// For every group in [group_begin, group_end), head h and j < count, the row
// kept_idx[j] of the source list is copied to row j of the destination list,
// for K and for V.  The index list of (group, head) is
// kept[(group*ipg + (ipg == 1 ? 0 : head))*kept_ld]; ipg = 1 is the shared
// draw.  count = kept_count[that index list] if kept_count is given, else K.
struct OracleStore {
  int paged;
  int64_t list_stride;
  const int32_t* page_table;
  int64_t pt_ld;
};

static int64_t row_offset(const OracleStore& st, int64_t group, int64_t t, int64_t head,
                          int32_t H, int32_t D, int32_t page_size) {
  if (!st.paged) return (group * H + head) * st.list_stride + t * D;
  int64_t page = st.page_table[group * st.pt_ld + t / page_size];
  return ((page * page_size + t % page_size) * H + head) * D;
}

void oracle_compact(int32_t src_paged, const uint16_t* k_src, const uint16_t* v_src,
                    int64_t src_list_stride, const int32_t* src_pt, int64_t src_pt_ld,
                    int32_t dst_paged, uint16_t* k_dst, uint16_t* v_dst, int64_t dst_list_stride,
                    const int32_t* dst_pt, int64_t dst_pt_ld, int32_t D, int32_t H,
                    int32_t page_size, const int32_t* kept, int64_t kept_ld,
                    const int32_t* kept_count, int32_t K, int64_t group_begin, int64_t group_end,
                    int32_t ipg) {
  OracleStore src{src_paged, src_list_stride, src_pt, src_pt_ld};
  OracleStore dst{dst_paged, dst_list_stride, dst_pt, dst_pt_ld};
  const size_t row_bytes = (size_t)D * 2;
  for (int64_t g = group_begin; g < group_end; ++g) {
    for (int32_t h = 0; h < H; ++h) {
      int64_t idx_list = g * ipg + (ipg == 1 ? 0 : h);
      int32_t count = kept_count ? kept_count[idx_list] : K;
      const int32_t* idx = kept + idx_list * kept_ld;
      for (int32_t j = 0; j < count; ++j) {
        int64_t so = row_offset(src, g, idx[j], h, H, D, page_size);
        int64_t dof = row_offset(dst, g, j, h, H, D, page_size);
        std::memcpy(k_dst + dof, k_src + so, row_bytes);
        std::memcpy(v_dst + dof, v_src + so, row_bytes);
      }
    }
  }
}

}  // extern "C"
