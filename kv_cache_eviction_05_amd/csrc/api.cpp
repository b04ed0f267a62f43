// C ABI of the eviction round: host-side validation and dispatch.
//
// Every entry point checks its arguments completely before enqueuing any
// work, so an error status means nothing was launched and no output touched.
// The library holds no state and allocates no memory.
#include <hip/hip_runtime.h>

#include <cfenv>
#include <cmath>
#include <cstdint>
#include <vector>

#include "kvevict.h"
#include "kvevict_launch.hpp"

namespace {

constexpr int64_t kInt32Max = 2147483647;
constexpr int64_t kUint32Max = 4294967295LL;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// a * b <= limit for a, b >= 0 and limit >= 0, decided without forming a
// product that could overflow.
bool prod_le(int64_t a, int64_t b, int64_t limit) { return a == 0 || b <= limit / a; }

// A launcher returns hipErrorInvalidConfiguration, before it enqueues anything, for a call too
// large for one grid (2^32 or more work-items in a dimension): a size out of its range.
kvevict_status hip_status(hipError_t e) {
  if (e == hipSuccess) return KVEVICT_OK;
  return e == hipErrorInvalidConfiguration ? KVEVICT_ERR_INVALID_ARG : KVEVICT_ERR_HIP;
}

int log2_exact(int32_t v) {
  if (v <= 0 || (v & (v - 1)) != 0) return -1;
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

// Validates one store description; fills the kernel's view of it.
kvevict_status check_store(const kvevict_kv_desc* d, const void* k, const void* v,
                           int64_t num_groups, kvevict::StoreView* out) {
  if (!d) return KVEVICT_ERR_INVALID_ARG;
  if (d->head_dim <= 0 || d->heads <= 0) return KVEVICT_ERR_INVALID_ARG;
  if (d->head_dim % 8 != 0) return KVEVICT_ERR_ALIGNMENT;
  if (num_groups > 0 && (!k || !v)) return KVEVICT_ERR_INVALID_ARG;
  if (!aligned16(k) || !aligned16(v)) return KVEVICT_ERR_ALIGNMENT;
  out->page_table = nullptr;
  out->pt_ld = 0;
  out->page_shift = 0;
  out->list_stride_v = 0;
  out->capacity = d->capacity;
  if (d->capacity < 0) return KVEVICT_ERR_INVALID_ARG;
  if (d->layout == KVEVICT_LAYOUT_CONTIG) {
    out->paged = 0;
    if (!prod_le(d->capacity, d->head_dim, INT64_MAX)) return KVEVICT_ERR_INVALID_ARG;
    if (d->list_stride < d->capacity * d->head_dim) return KVEVICT_ERR_INVALID_ARG;
    if (d->list_stride % 8 != 0) return KVEVICT_ERR_ALIGNMENT;
    out->list_stride_v = d->list_stride / 8;
    out->max_rows = d->capacity;
  } else if (d->layout == KVEVICT_LAYOUT_PAGED) {
    out->paged = 1;
    if (d->page_size <= 0 || d->pt_ld <= 0) return KVEVICT_ERR_INVALID_ARG;
    const int shift = log2_exact(d->page_size);
    if (shift < 0) return KVEVICT_ERR_UNSUPPORTED;  // page sizes are powers of two
    if (num_groups > 0 && !d->page_table) return KVEVICT_ERR_INVALID_ARG;
    if (d->pt_ld > (kInt32Max >> shift)) return KVEVICT_ERR_INVALID_ARG;
    out->page_shift = shift;
    out->page_table = d->page_table;
    out->pt_ld = d->pt_ld;
    out->max_rows = d->pt_ld << shift;
  } else {
    return KVEVICT_ERR_INVALID_ARG;
  }
  return KVEVICT_OK;
}

// Byte extent of a store as its descriptor lays it out for `lists` lists:
// contiguous ((lists - 1)*list_stride + capacity*D) elements, paged
// capacity*page_size*H*D elements (the whole pool), 2 bytes each.  Taken in
// 128-bit arithmetic on a validated descriptor, so it cannot wrap.
typedef unsigned __int128 u128;
u128 store_extent_bytes(const kvevict_kv_desc* d, int64_t lists) {
  if (lists <= 0) return 0;
  u128 elems;
  if (d->layout == KVEVICT_LAYOUT_CONTIG)
    elems = (u128)(lists - 1) * (u128)d->list_stride + (u128)d->capacity * (u128)d->head_dim;
  else
    elems = (u128)d->capacity * (u128)d->page_size * (u128)d->heads * (u128)d->head_dim;
  return elems * 2u;
}

// True if the byte ranges [a, a + alen) and [b, b + blen) share a byte.
bool ranges_overlap(const void* a, u128 alen, const void* b, u128 blen) {
  if (alen == 0 || blen == 0) return false;
  const u128 x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + blen && y < x + alen;
}

}  // namespace

extern "C" {

kvevict_status kvevict_score_random(float* scores, int64_t ld, int64_t num_requests, int32_t L,
                                    int32_t H, int32_t n, int32_t prot, uint64_t seed,
                                    uint32_t round, int32_t shared_draw, hipStream_t stream) {
  if (num_requests < 0 || num_requests > 0xffffffffll || L < 1 || H < 1) return KVEVICT_ERR_INVALID_ARG;
  if (n < 0 || prot < 0 || prot > n || ld < n) return KVEVICT_ERR_INVALID_ARG;
  const int64_t per_request = (int64_t)L * (shared_draw ? 1 : H);
  if (!prod_le(num_requests, per_request, kInt32Max)) return KVEVICT_ERR_INVALID_ARG;
  const int64_t lists = num_requests * per_request;
  if (lists > 0 && n > 0 && !scores) return KVEVICT_ERR_INVALID_ARG;
  return hip_status(kvevict::launch_score_random(scores, ld, lists, L, H, n, prot, seed, round,
                                                 shared_draw != 0, stream));
}

// Arguments of the weighted score (kvevict_score_weighted and the fused score +
// global top-B), with the windows copied into *win.
static kvevict_status check_weighted(const float* scores, int64_t ld, const float* beta,
                                     const float* vnorm, int64_t sig_stride_g,
                                     int64_t sig_stride_t, int64_t sig_stride_j, const float* w,
                                     int32_t w_slots, const int32_t* win_begin,
                                     const int32_t* win_count, int32_t L, int32_t H, int32_t G,
                                     int32_t Hg, int32_t n, int32_t prot,
                                     kvevict::WindowTable* win) {
  if (L < 1 || L > kvevict::kMaxWeightedLayers || H < 1 || G < 1 || Hg < 1) return KVEVICT_ERR_INVALID_ARG;
  if (n < 0 || prot < 0 || prot > n || ld < n) return KVEVICT_ERR_INVALID_ARG;
  if (w_slots < 1 || w_slots > 64) return KVEVICT_ERR_INVALID_ARG;
  if (!win_begin || !win_count) return KVEVICT_ERR_INVALID_ARG;
  if (sig_stride_g < 0 || sig_stride_t < 0 || sig_stride_j < 0) return KVEVICT_ERR_INVALID_ARG;
  for (int32_t l = 0; l < L; ++l) {
    if (win_count[l] < 0 || win_count[l] > w_slots) return KVEVICT_ERR_INVALID_ARG;
    if (win_begin[l] < 0 || win_begin[l] + (int64_t)win_count[l] > G) return KVEVICT_ERR_INVALID_ARG;
    win->begin[l] = win_begin[l];
    win->count[l] = win_count[l];
  }
  if (n > 0 && (!scores || !beta || !vnorm || !w)) return KVEVICT_ERR_INVALID_ARG;
  return KVEVICT_OK;
}

kvevict_status kvevict_score_weighted(float* scores, int64_t ld, const float* beta,
                                      const float* vnorm, int64_t sig_stride_g,
                                      int64_t sig_stride_t, int64_t sig_stride_j, const float* w,
                                      int32_t w_slots, const int32_t* win_begin,
                                      const int32_t* win_count, int32_t L, int32_t H, int32_t G,
                                      int32_t Hg, int32_t n, int32_t prot, hipStream_t stream) {
  kvevict::WindowTable win;
  const kvevict_status st = check_weighted(scores, ld, beta, vnorm, sig_stride_g, sig_stride_t,
                                           sig_stride_j, w, w_slots, win_begin, win_count, L, H,
                                           G, Hg, n, prot, &win);
  if (st != KVEVICT_OK) return st;
  return hip_status(kvevict::launch_score_weighted(scores, ld, beta, vnorm, sig_stride_g,
                                                   sig_stride_t, sig_stride_j, w, w_slots, win, L,
                                                   H, Hg, n, prot, stream));
}

kvevict_status kvevict_select_topk(int32_t* kept_idx, int64_t kept_ld, const float* scores,
                                   int64_t ld, int64_t num_lists, int32_t n, int32_t K,
                                   int32_t prot, hipStream_t stream) {
  if (num_lists < 0 || num_lists > kInt32Max) return KVEVICT_ERR_INVALID_ARG;
  if (prot < 0 || K < prot || n < K || ld < n || kept_ld < K) return KVEVICT_ERR_INVALID_ARG;
  if (num_lists > 0 && K > 0 && (!kept_idx || !scores)) return KVEVICT_ERR_INVALID_ARG;
  return hip_status(kvevict::launch_select_topk(kept_idx, kept_ld, nullptr, scores, ld, num_lists,
                                                n, K, prot, 0, 1, nullptr, stream));
}

kvevict_status kvevict_score_keydiff(float* scores, int64_t ld, const kvevict_kv_desc* keys,
                                     const void* k_cache, int64_t num_groups, int32_t n,
                                     int32_t prot, hipStream_t stream) {
  if (!keys || num_groups < 0 || n < 0 || prot < 0 || prot > n || ld < n) return KVEVICT_ERR_INVALID_ARG;
  const int32_t D = keys->head_dim, H = keys->heads;
  kvevict::StoreView sv;
  const kvevict_status st = check_store(keys, k_cache, k_cache, num_groups, &sv);
  if (st != KVEVICT_OK) return st;
  const int32_t vpr = D / 8;
  if (vpr > 64 || (vpr & (vpr - 1)) != 0) return KVEVICT_ERR_UNSUPPORTED;  // D in {8, 16, ..., 512}
  if (n > sv.max_rows) return KVEVICT_ERR_INVALID_ARG;
  if ((int64_t)n * vpr > kInt32Max) return KVEVICT_ERR_INVALID_ARG;  // 32-bit row offsets
  // one workgroup of up to 512 threads per list, fewer than 2^32 work-items per launch
  if (!prod_le(num_groups, H, (1LL << 23) - 1)) return KVEVICT_ERR_INVALID_ARG;
  const int64_t lists = num_groups * H;
  if (lists > 0 && n > 0 && !scores) return KVEVICT_ERR_INVALID_ARG;
  return hip_status(kvevict::launch_score_keydiff(scores, ld, sv, k_cache, D, H, lists, n, prot,
                                                  stream));
}

kvevict_status kvevict_select_topk_layers(int32_t* kept_idx, int64_t kept_ld,
                                          int32_t* kept_count, const float* scores, int64_t ld,
                                          int64_t num_groups, int32_t L, int32_t H, int32_t n,
                                          int32_t prot, const int32_t* layer_budget,
                                          hipStream_t stream) {
  if (num_groups < 0 || L < 1 || L > kvevict::kMaxBudgetLayers || H < 1) return KVEVICT_ERR_INVALID_ARG;
  if (num_groups % L != 0) return KVEVICT_ERR_INVALID_ARG;  // whole requests of L layers
  if (prot < 0 || n < prot || ld < n || !layer_budget) return KVEVICT_ERR_INVALID_ARG;
  int32_t most = 0;
  for (int32_t l = 0; l < L; ++l) {
    if (layer_budget[l] < 0 || layer_budget[l] > n - prot) return KVEVICT_ERR_INVALID_ARG;
    most = layer_budget[l] > most ? layer_budget[l] : most;
  }
  if (kept_ld < prot + most) return KVEVICT_ERR_INVALID_ARG;
  if (!prod_le(num_groups, H, kInt32Max)) return KVEVICT_ERR_INVALID_ARG;
  const int64_t lists = num_groups * H;
  if (lists > 0 && (!kept_idx || !kept_count || !scores)) return KVEVICT_ERR_INVALID_ARG;
  return hip_status(kvevict::launch_select_topk(kept_idx, kept_ld, kept_count, scores, ld, lists,
                                                n, prot, prot, L, H, layer_budget, stream));
}

kvevict_status kvevict_reduce_max_heads(float* shared, int64_t shared_ld, const float* scores,
                                        int64_t ld, int64_t num_groups, int32_t H, int32_t n,
                                        hipStream_t stream) {
  if (num_groups < 0 || H < 1 || n < 0 || ld < n || shared_ld < n) return KVEVICT_ERR_INVALID_ARG;
  if (!prod_le(num_groups, H, kInt32Max)) return KVEVICT_ERR_INVALID_ARG;
  if (num_groups > 0 && n > 0 && (!shared || !scores)) return KVEVICT_ERR_INVALID_ARG;
  return hip_status(
      kvevict::launch_reduce_max_heads(shared, shared_ld, scores, ld, num_groups, H, n, stream));
}

kvevict_status kvevict_layer_power_budget(const float* gate, int32_t L, int32_t n_body, double p,
                                          int32_t* budget) {
  // Exact arithmetic on the float gates: gate_l = m_l * 2^e_l with m_l < 2^24, scaled
  // to integers w_l = m_l * 2^(e_l - e_min) (gates may span at most 2^40).
  if (!gate || !budget || L < 1 || L > 4096 || n_body < 0) return KVEVICT_ERR_INVALID_ARG;
  if (!(p >= 0.0 && p <= 1.0)) return KVEVICT_ERR_INVALID_ARG;
  typedef unsigned __int128 u128;
  std::vector<uint32_t> mant(L);
  std::vector<int> expo(L);
  int emin = 1 << 30, emax = -(1 << 30);
  for (int32_t l = 0; l < L; ++l) {
    const float g = gate[l];
    if (!(g > 0.0f) || !std::isfinite(g)) return KVEVICT_ERR_INVALID_ARG;
    int e = 0;
    const float f = std::frexp(g, &e);  // g = f * 2^e, f in [0.5, 1)
    mant[l] = (uint32_t)std::ldexp(f, 24);
    expo[l] = e - 24;
    emin = expo[l] < emin ? expo[l] : emin;
    emax = expo[l] > emax ? expo[l] : emax;
  }
  if (emax - emin > 40) return KVEVICT_ERR_INVALID_ARG;
  std::vector<u128> w(L);
  for (int32_t l = 0; l < L; ++l) w[l] = (u128)mant[l] << (expo[l] - emin);
  // flat per-list budget round(p * n_body): binary64 product, ties to even
  const int saved = std::fegetround();
  std::fesetround(FE_TONEAREST);
  const int64_t flat = (int64_t)std::nearbyint(p * (double)n_body);
  std::fesetround(saved);
  const int64_t T = (int64_t)L * flat;
  // layers whose proportional share passes n_body are capped there; the rest share what is left
  std::vector<char> capped(L, 0);
  int64_t ncap = 0;
  u128 S = 0;
  int64_t T2 = T;
  for (;;) {
    S = 0;
    for (int32_t l = 0; l < L; ++l)
      if (!capped[l]) S += w[l];
    T2 = T - ncap * (int64_t)n_body;
    bool more = false;
    for (int32_t l = 0; l < L; ++l) {
      if (!capped[l] && (u128)T2 * w[l] > (u128)n_body * S) {
        capped[l] = 1;
        ++ncap;
        more = true;
      }
    }
    if (!more) break;
  }
  // floors of the shares, then one more for the largest remainders (ties: lower layer)
  std::vector<u128> rem(L, 0);
  int64_t given = 0;
  for (int32_t l = 0; l < L; ++l) {
    if (capped[l]) {
      budget[l] = n_body;
    } else {
      const u128 q = (u128)T2 * w[l];
      budget[l] = (int32_t)(q / S);
      rem[l] = q % S;
    }
    given += budget[l];
  }
  for (int64_t left = T - given; left > 0; --left) {
    int32_t pick = -1;
    for (int32_t l = 0; l < L; ++l)
      if (!capped[l] && rem[l] != (u128)-1 && (pick < 0 || rem[l] > rem[pick])) pick = l;
    if (pick < 0) return KVEVICT_ERR_INVALID_ARG;  // unreachable: T <= L * n_body
    budget[pick] += 1;
    rem[pick] = (u128)-1;  // taken
  }
  return KVEVICT_OK;
}

// Arguments, workspace protocol and budget of a global top-B over num_lists
// lists of n scores (kvevict_select_global and the fused score + global top-B).
// *launch is false when the call only reports the workspace size.
static kvevict_status check_global(int32_t* kept_idx, int64_t kept_ld, int32_t* kept_count,
                                   int64_t ld, int64_t num_lists, int32_t n, int32_t prot,
                                   double p, void* workspace, size_t* workspace_bytes,
                                   int64_t* budget, bool* launch) {
  *launch = false;
  if (!workspace_bytes) return KVEVICT_ERR_INVALID_ARG;
  if (num_lists < 0 || n < 0 || prot < 0 || prot > n || ld < n || kept_ld < n) return KVEVICT_ERR_INVALID_ARG;
  if (!(p >= 0.0 && p <= 1.0)) return KVEVICT_ERR_INVALID_ARG;  // also rejects NaN
  if (!prod_le(num_lists, n, kInt32Max)) return KVEVICT_ERR_INVALID_ARG;
  const size_t need = kvevict::select_global_workspace_bytes(num_lists, n, prot);
  if (!workspace) {
    *workspace_bytes = need;
    return KVEVICT_OK;
  }
  if (*workspace_bytes < need) return KVEVICT_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 3u) return KVEVICT_ERR_ALIGNMENT;
  if (num_lists > 0 && (!kept_idx || !kept_count)) return KVEVICT_ERR_INVALID_ARG;
  // B = lists * round(p * (n - prot)): binary64 product, ties to even.
  const int saved = std::fegetround();
  std::fesetround(FE_TONEAREST);
  const double per_list = std::nearbyint(p * (double)(n - prot));
  std::fesetround(saved);
  *budget = num_lists * (int64_t)per_list;
  *launch = true;
  return KVEVICT_OK;
}

kvevict_status kvevict_select_global(int32_t* kept_idx, int64_t kept_ld, int32_t* kept_count,
                                     int64_t* budget_out, const float* scores, int64_t ld,
                                     int64_t num_lists, int32_t n, int32_t prot, double p,
                                     void* workspace, size_t* workspace_bytes,
                                     hipStream_t stream) {
  int64_t budget = 0;
  bool launch = false;
  const kvevict_status st = check_global(kept_idx, kept_ld, kept_count, ld, num_lists, n, prot, p,
                                         workspace, workspace_bytes, &budget, &launch);
  if (st != KVEVICT_OK || !launch) return st;
  if (num_lists > 0 && !scores) return KVEVICT_ERR_INVALID_ARG;
  if (num_lists > kvevict::max_workgroups(kvevict::kGlobalThreads)) return KVEVICT_ERR_INVALID_ARG;
  if (budget_out) *budget_out = budget;
  return hip_status(kvevict::launch_select_global(kept_idx, kept_ld, kept_count, scores, ld,
                                                  num_lists, n, prot, budget, workspace, stream));
}

kvevict_status kvevict_select_global_noalloc(int32_t* kept_idx, int64_t kept_ld,
                                             int32_t* kept_count, int64_t* budget_out,
                                             const float* scores, int64_t ld, int64_t num_lists,
                                             int32_t n, int32_t prot, double p,
                                             hipStream_t stream) {
  // the arguments, and the workspace the call needs against the static array's size
  size_t need = 0;
  int64_t budget = 0;
  bool launch = false;
  kvevict_status st = check_global(kept_idx, kept_ld, kept_count, ld, num_lists, n, prot, p,
                                   nullptr, &need, &budget, &launch);
  if (st != KVEVICT_OK) return st;
  if (need > (size_t)KVEVICT_SELECT_GLOBAL_NOALLOC_BYTES) return KVEVICT_ERR_WORKSPACE;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (kvevict::select_global_scratch(&ws, &ws_bytes) != hipSuccess) return KVEVICT_ERR_HIP;
  st = check_global(kept_idx, kept_ld, kept_count, ld, num_lists, n, prot, p, ws, &ws_bytes,
                    &budget, &launch);
  if (st != KVEVICT_OK || !launch) return st;
  if (num_lists > 0 && !scores) return KVEVICT_ERR_INVALID_ARG;
  if (num_lists > kvevict::max_workgroups(kvevict::kGlobalThreads)) return KVEVICT_ERR_INVALID_ARG;
  if (budget_out) *budget_out = budget;
  return hip_status(kvevict::launch_select_global(kept_idx, kept_ld, kept_count, scores, ld,
                                                  num_lists, n, prot, budget, ws, stream));
}

kvevict_status kvevict_score_select_global(
    int32_t* kept_idx, int64_t kept_ld, int32_t* kept_count, int64_t* budget_out, float* scores,
    int64_t ld, const float* beta, const float* vnorm, int64_t sig_stride_g,
    int64_t sig_stride_t, int64_t sig_stride_j, const float* w, int32_t w_slots,
    const int32_t* win_begin, const int32_t* win_count, int32_t L, int32_t H, int32_t G,
    int32_t Hg, int32_t n, int32_t prot, double p, void* workspace, size_t* workspace_bytes,
    hipStream_t stream) {
  kvevict::WindowTable win;
  kvevict_status st = check_weighted(scores, ld, beta, vnorm, sig_stride_g, sig_stride_t,
                                     sig_stride_j, w, w_slots, win_begin, win_count, L, H, G, Hg,
                                     n, prot, &win);
  if (st != KVEVICT_OK) return st;
  const int64_t num_lists = (int64_t)L * H;
  int64_t budget = 0;
  bool launch = false;
  st = check_global(kept_idx, kept_ld, kept_count, ld, num_lists, n, prot, p, workspace,
                    workspace_bytes, &budget, &launch);
  if (st != KVEVICT_OK || !launch) return st;
  // every launch of the call fits its grid before the first is enqueued (and before any
  // output is written)
  if (num_lists > kvevict::max_workgroups(kvevict::kGlobalThreads) ||
      (n + kvevict::kWeightedTile - 1) / kvevict::kWeightedTile >
          kvevict::max_workgroups(kvevict::kWeightedThreads))
    return KVEVICT_ERR_INVALID_ARG;
  if (budget_out) *budget_out = budget;
  // prompts and cleared workspace, then the scores with the first radix level
  // added by the scorer, then the rest of the select
  hipError_t e = kvevict::launch_select_global_init(kept_idx, kept_ld, kept_count, num_lists, n,
                                                    prot, budget, workspace, stream);
  if (e != hipSuccess) return hip_status(e);
  uint32_t* bins = kvevict::select_global_first_level_bins(num_lists, n, prot, budget, workspace);
  e = kvevict::launch_score_weighted(scores, ld, beta, vnorm, sig_stride_g, sig_stride_t,
                                     sig_stride_j, w, w_slots, win, L, H, Hg, n, prot, stream,
                                     bins);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(kvevict::launch_select_global(kept_idx, kept_ld, kept_count, scores, ld,
                                                  num_lists, n, prot, budget, workspace, stream,
                                                  true));
}

// Arguments of an out-of-place compaction: the two stores' views, K within
// the destination, and no destination byte inside a source or the other
// destination (the sources are only read and may overlap).
static kvevict_status check_compact(const kvevict_kv_desc* src, const void* k_src,
                                    const void* v_src, const kvevict_kv_desc* dst,
                                    const void* k_dst, const void* v_dst,
                                    const int32_t* kept_idx, int64_t kept_ld, int32_t K,
                                    int64_t num_groups, int32_t idx_lists_per_group,
                                    kvevict::StoreView* sv, kvevict::StoreView* dv) {
  if (!src || !dst) return KVEVICT_ERR_INVALID_ARG;
  if (num_groups < 0 || K < 0 || kept_ld < K) return KVEVICT_ERR_INVALID_ARG;
  if (src->head_dim != dst->head_dim || src->heads != dst->heads) return KVEVICT_ERR_INVALID_ARG;
  const int32_t H = src->heads;
  if (idx_lists_per_group != 1 && idx_lists_per_group != H) return KVEVICT_ERR_INVALID_ARG;
  kvevict_status st = check_store(src, k_src, v_src, num_groups, sv);
  if (st != KVEVICT_OK) return st;
  st = check_store(dst, k_dst, v_dst, num_groups, dv);
  if (st != KVEVICT_OK) return st;
  if (K > dv->max_rows) return KVEVICT_ERR_INVALID_ARG;
  if (!prod_le(num_groups, H, kInt32Max)) return KVEVICT_ERR_INVALID_ARG;
  if (num_groups > 0 && K > 0 && !kept_idx) return KVEVICT_ERR_INVALID_ARG;
  const int32_t D = src->head_dim;
  if ((int64_t)H * D > (1 << 26)) return KVEVICT_ERR_INVALID_ARG;  // one token row of all heads
  if (num_groups > 0 && K > 0) {
    const int64_t lists = num_groups * H;
    const u128 se = store_extent_bytes(src, lists), de = store_extent_bytes(dst, lists);
    if (ranges_overlap(k_dst, de, k_src, se) || ranges_overlap(k_dst, de, v_src, se) ||
        ranges_overlap(v_dst, de, k_src, se) || ranges_overlap(v_dst, de, v_src, se) ||
        ranges_overlap(k_dst, de, v_dst, de))
      return KVEVICT_ERR_INVALID_ARG;
  }
  return KVEVICT_OK;
}

kvevict_status kvevict_compact(const kvevict_kv_desc* src, const void* k_src, const void* v_src,
                               const kvevict_kv_desc* dst, void* k_dst, void* v_dst,
                               const int32_t* kept_idx, int64_t kept_ld,
                               const int32_t* kept_count, int32_t K, int64_t num_groups,
                               int32_t idx_lists_per_group, uint32_t* errors,
                               hipStream_t stream) {
  kvevict::StoreView sv, dv;
  const kvevict_status st = check_compact(src, k_src, v_src, dst, k_dst, v_dst, kept_idx, kept_ld,
                                          K, num_groups, idx_lists_per_group, &sv, &dv);
  if (st != KVEVICT_OK) return st;
  return hip_status(kvevict::launch_compact(sv, k_src, v_src, dv, k_dst, v_dst, src->head_dim,
                                            src->heads, kept_idx, kept_ld, kept_count, K,
                                            num_groups, idx_lists_per_group, errors, stream));
}

kvevict_status kvevict_compact_ordered(const kvevict_kv_desc* src, const void* k_src,
                                       const void* v_src, const kvevict_kv_desc* dst,
                                       void* k_dst, void* v_dst, const int32_t* kept_idx,
                                       int64_t kept_ld, const int32_t* kept_count, int32_t K,
                                       int64_t num_groups, int32_t idx_lists_per_group,
                                       uint32_t* errors, void* workspace,
                                       size_t* workspace_bytes, hipStream_t stream) {
  if (!workspace_bytes) return KVEVICT_ERR_INVALID_ARG;
  if (!dst) return KVEVICT_ERR_INVALID_ARG;
  if (!workspace) {  // size query: the destination pool's pages as int32 slots, and a flag
    if (dst->layout == KVEVICT_LAYOUT_PAGED) {
      if (dst->capacity < 0 || dst->capacity > (INT64_MAX - 512) / 4) return KVEVICT_ERR_INVALID_ARG;
      kvevict::StoreView dv{};
      dv.capacity = dst->capacity;
      *workspace_bytes = kvevict::compact_order_workspace_bytes(dv);
    } else {
      *workspace_bytes = 0;
    }
    return KVEVICT_OK;
  }
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return KVEVICT_ERR_ALIGNMENT;
  if (dst->layout == KVEVICT_LAYOUT_PAGED) {
    kvevict::StoreView dv{};
    dv.capacity = dst->capacity < 0 ? 0 : dst->capacity;
    if (*workspace_bytes < kvevict::compact_order_workspace_bytes(dv)) return KVEVICT_ERR_WORKSPACE;
  }
  kvevict::StoreView sv, dv;
  const kvevict_status st = check_compact(src, k_src, v_src, dst, k_dst, v_dst, kept_idx, kept_ld,
                                          K, num_groups, idx_lists_per_group, &sv, &dv);
  if (st != KVEVICT_OK) return st;
  if (dv.paged && num_groups > 0 && K > 0) {  // the workspace is written: apart from the stores
    const int64_t lists = num_groups * src->heads;
    const u128 wext = (u128)kvevict::compact_order_workspace_bytes(dv);
    const u128 se = store_extent_bytes(src, lists), de = store_extent_bytes(dst, lists);
    if (ranges_overlap(workspace, wext, k_src, se) || ranges_overlap(workspace, wext, v_src, se) ||
        ranges_overlap(workspace, wext, k_dst, de) || ranges_overlap(workspace, wext, v_dst, de))
      return KVEVICT_ERR_INVALID_ARG;
  }
  return hip_status(kvevict::launch_compact(sv, k_src, v_src, dv, k_dst, v_dst, src->head_dim,
                                            src->heads, kept_idx, kept_ld, kept_count, K,
                                            num_groups, idx_lists_per_group, errors, stream,
                                            dv.paged ? workspace : nullptr));
}

kvevict_status kvevict_copy_pages(const void* k_src, const void* v_src, int64_t src_pages,
                                  const int32_t* src_ids, void* k_dst, void* v_dst,
                                  int64_t dst_pages, const int32_t* dst_ids, int64_t count,
                                  int64_t page_bytes, uint32_t* errors, hipStream_t stream) {
  if (count < 0 || src_pages < 0 || dst_pages < 0) return KVEVICT_ERR_INVALID_ARG;
  if (page_bytes <= 0) return KVEVICT_ERR_INVALID_ARG;
  if (page_bytes % 16 != 0) return KVEVICT_ERR_ALIGNMENT;
  if (count == 0) return KVEVICT_OK;
  if (!k_src || !v_src || !k_dst || !v_dst || !src_ids || !dst_ids) return KVEVICT_ERR_INVALID_ARG;
  if (!aligned16(k_src) || !aligned16(v_src) || !aligned16(k_dst) || !aligned16(v_dst))
    return KVEVICT_ERR_ALIGNMENT;
  if (!prod_le(src_pages, page_bytes, INT64_MAX) || !prod_le(dst_pages, page_bytes, INT64_MAX))
    return KVEVICT_ERR_INVALID_ARG;
  const u128 se = (u128)src_pages * (u128)page_bytes, de = (u128)dst_pages * (u128)page_bytes;
  if (ranges_overlap(k_dst, de, k_src, se) || ranges_overlap(k_dst, de, v_src, se) ||
      ranges_overlap(v_dst, de, k_src, se) || ranges_overlap(v_dst, de, v_src, se) ||
      ranges_overlap(k_dst, de, v_dst, de))
    return KVEVICT_ERR_INVALID_ARG;
  return hip_status(kvevict::launch_copy_pages(k_src, v_src, src_pages, src_ids, k_dst, v_dst,
                                               dst_pages, dst_ids, count, page_bytes, errors,
                                               stream));
}

kvevict_status kvevict_compact_inplace(const kvevict_kv_desc* store, void* k, void* v,
                                       const int32_t* kept_idx, int64_t kept_ld,
                                       const int32_t* kept_count, int32_t K, int32_t n,
                                       int64_t num_groups, int32_t idx_lists_per_group,
                                       int32_t* freed_pages, uint32_t* freed_count,
                                       uint32_t* errors, hipStream_t stream) {
  if (!store) return KVEVICT_ERR_INVALID_ARG;
  if (num_groups < 0 || K < 0 || n < K || kept_ld < K) return KVEVICT_ERR_INVALID_ARG;
  const int32_t H = store->heads, D = store->head_dim;
  if (idx_lists_per_group != 1 && idx_lists_per_group != H) return KVEVICT_ERR_INVALID_ARG;
  kvevict::StoreView sv;
  const kvevict_status st = check_store(store, k, v, num_groups, &sv);
  if (st != KVEVICT_OK) return st;
  if ((int64_t)H * D > (1 << 26)) return KVEVICT_ERR_INVALID_ARG;
  if (n > sv.max_rows) return KVEVICT_ERR_INVALID_ARG;
  if (num_groups > 0 && K > 0 && !kept_idx) return KVEVICT_ERR_INVALID_ARG;
  if (sv.paged && num_groups > 0 && (!freed_pages || !freed_count)) return KVEVICT_ERR_INVALID_ARG;
  if (!prod_le(num_groups, H, kInt32Max) || (int64_t)n * (D / 8) > (1LL << 30)) return KVEVICT_ERR_INVALID_ARG;
  if (num_groups > 0 && ranges_overlap(k, store_extent_bytes(store, num_groups * H), v,
                                       store_extent_bytes(store, num_groups * H)))
    return KVEVICT_ERR_INVALID_ARG;  // K and V are disjoint stores
  if (sv.paged && !prod_le(num_groups, (n + store->page_size - 1) / store->page_size, kUint32Max))
    return KVEVICT_ERR_INVALID_ARG;  // free-list offsets are 32-bit
  return hip_status(kvevict::launch_compact_inplace(sv, k, v, D, H, kept_idx, kept_ld, kept_count,
                                                    K, n, num_groups, idx_lists_per_group,
                                                    sv.paged ? freed_pages : nullptr,
                                                    freed_count, errors, stream));
}

kvevict_status kvevict_evict_random_inplace(const kvevict_kv_desc* store, void* k, void* v,
                                           int64_t num_requests, int32_t L, int32_t n, int32_t K,
                                           int32_t prot, uint64_t seed, uint32_t round,
                                           int32_t shared_draw, int32_t* kept_idx,
                                           int64_t kept_ld, int32_t* freed_pages,
                                           uint32_t* freed_count, uint32_t* errors,
                                           hipStream_t stream) {
  if (!store) return KVEVICT_ERR_INVALID_ARG;
  if (num_requests < 0 || num_requests > 0xffffffffll || L < 1) return KVEVICT_ERR_INVALID_ARG;
  if (prot < 0 || K < prot || n < K) return KVEVICT_ERR_INVALID_ARG;
  if (kept_idx && kept_ld < K) return KVEVICT_ERR_INVALID_ARG;
  const int64_t num_groups = num_requests * L;
  const int32_t H = store->heads, D = store->head_dim;
  kvevict::StoreView sv;
  const kvevict_status st = check_store(store, k, v, num_groups, &sv);
  if (st != KVEVICT_OK) return st;
  if ((int64_t)H * D > (1 << 26)) return KVEVICT_ERR_INVALID_ARG;
  if (n > sv.max_rows) return KVEVICT_ERR_INVALID_ARG;
  if (sv.paged && num_groups > 0 && (!freed_pages || !freed_count)) return KVEVICT_ERR_INVALID_ARG;
  if (!prod_le(num_groups, H, kInt32Max) || (int64_t)n * (D / 8) > (1LL << 30)) return KVEVICT_ERR_INVALID_ARG;
  if (num_groups > 0 && ranges_overlap(k, store_extent_bytes(store, num_groups * H), v,
                                       store_extent_bytes(store, num_groups * H)))
    return KVEVICT_ERR_INVALID_ARG;  // K and V are disjoint stores
  if ((int64_t)(n - prot) + K > kvevict::kMaxFusedEntries) return KVEVICT_ERR_UNSUPPORTED;
  if (sv.paged && !prod_le(num_groups, (n + store->page_size - 1) / store->page_size, kUint32Max))
    return KVEVICT_ERR_INVALID_ARG;  // free-list offsets are 32-bit
  return hip_status(kvevict::launch_evict_random_inplace(
      sv, k, v, D, H, num_groups, L, n, K, prot, seed, round, shared_draw != 0, kept_idx, kept_ld,
      sv.paged ? freed_pages : nullptr, freed_count, errors, stream));
}

kvevict_status kvevict_select_random(int32_t* kept_idx, int64_t kept_ld, int64_t num_requests,
                                     int32_t L, int32_t H, int32_t n, int32_t K, int32_t prot,
                                     uint64_t seed, uint32_t round, int32_t shared_draw,
                                     hipStream_t stream) {
  if (num_requests < 0 || num_requests > 0xffffffffll || L < 1 || H < 1) return KVEVICT_ERR_INVALID_ARG;
  if (prot < 0 || K < prot || n < K || kept_ld < K) return KVEVICT_ERR_INVALID_ARG;
  const int64_t per_request = (int64_t)L * (shared_draw ? 1 : H);
  if (!prod_le(num_requests, per_request, kInt32Max)) return KVEVICT_ERR_INVALID_ARG;
  const int64_t lists = num_requests * per_request;
  if (lists > 0 && K > 0 && !kept_idx) return KVEVICT_ERR_INVALID_ARG;
  return hip_status(kvevict::launch_draw_select(kept_idx, kept_ld, lists, L, H, n, K, prot, seed,
                                                round, shared_draw != 0, stream));
}

kvevict_status kvevict_evict_pages_random(int32_t* page_table, int64_t pt_ld, int32_t page_size,
                                         int64_t num_requests, int32_t L, int32_t n, int32_t K,
                                         int32_t prot, uint64_t seed, uint32_t round,
                                         int32_t* kept_pages, int64_t kept_ld,
                                         int32_t* freed_pages, uint32_t* freed_count,
                                         hipStream_t stream) {
  if (num_requests < 0 || num_requests > 0xffffffffll || L < 1) return KVEVICT_ERR_INVALID_ARG;
  if (page_size < 1 || prot < 0 || K < prot || n < K) return KVEVICT_ERR_INVALID_ARG;
  if (n % page_size != 0 || K % page_size != 0) return KVEVICT_ERR_INVALID_ARG;
  const int64_t num_groups = num_requests * L;
  if (num_groups > kInt32Max) return KVEVICT_ERR_INVALID_ARG;
  const int32_t P = n / page_size, Kp = K / page_size, pp = (prot + page_size - 1) / page_size;
  if (pt_ld < P) return KVEVICT_ERR_INVALID_ARG;
  if (kept_pages && kept_ld < Kp) return KVEVICT_ERR_INVALID_ARG;
  if (num_groups > 0 && (!page_table || !freed_pages || !freed_count)) return KVEVICT_ERR_INVALID_ARG;
  if (num_groups * (int64_t)(P - Kp) > kUint32Max) return KVEVICT_ERR_INVALID_ARG;  // 32-bit offsets
  if (kvevict::evict_pages_lds_bytes(P, pp, Kp) > (size_t)kvevict::kMaxFusedEntries * 4)
    return KVEVICT_ERR_UNSUPPORTED;
  return hip_status(kvevict::launch_evict_pages(page_table, pt_ld, page_size, num_groups, L, n, K,
                                                prot, seed, round, kept_pages, kept_ld,
                                                freed_pages, freed_count, stream));
}

const char* kvevict_status_string(kvevict_status status) {
  switch (status) {
    case KVEVICT_OK: return "ok";
    case KVEVICT_ERR_INVALID_ARG: return "invalid argument";
    case KVEVICT_ERR_ALIGNMENT: return "misaligned K/V base, stride or head_dim";
    case KVEVICT_ERR_WORKSPACE: return "workspace missing or too small";
    case KVEVICT_ERR_UNSUPPORTED: return "unsupported request";
    case KVEVICT_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int32_t kvevict_abi_version(void) { return KVEVICT_ABI_VERSION; }

}  // extern "C"
