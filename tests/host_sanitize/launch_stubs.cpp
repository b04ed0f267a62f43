// Stand-ins for the kernel launchers, for building the C ABI's host code
// (api.cpp) with g++ under AddressSanitizer and UndefinedBehaviorSanitizer.
// Each launcher counts its call and checks the sizes that api.cpp's
// validation promises every launcher; it launches nothing.
#include <cstdio>
#include <cstdlib>

#include "kvevict_launch.hpp"

int g_launches = 0;

namespace {
void need(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "launcher reached with unvalidated arguments: %s\n", what);
    std::abort();
  }
}
hipError_t launched() {
  ++g_launches;
  return hipSuccess;
}
}  // namespace

namespace kvevict {

hipError_t launch_score_random(float* scores, int64_t ld, int64_t num_lists, int32_t, int32_t,
                               int32_t n, int32_t prot, uint64_t, uint32_t, bool, hipStream_t) {
  need(num_lists >= 0 && num_lists <= 2147483647 && n >= 0 && prot >= 0 && prot <= n && ld >= n,
       "score_random sizes");
  need(num_lists == 0 || n == 0 || scores, "score_random pointer");
  return launched();
}

hipError_t launch_score_weighted(float* scores, int64_t ld, const float*, const float*, int64_t,
                                 int64_t, int64_t, const float*, int32_t w_slots,
                                 const WindowTable&, int32_t L, int32_t H, int32_t Hg, int32_t n,
                                 int32_t prot, hipStream_t, uint32_t*) {
  need(L >= 1 && L <= kMaxWeightedLayers && H >= 1 && Hg >= 1 && w_slots >= 1 && n >= 0 &&
           prot >= 0 && prot <= n && ld >= n && (n == 0 || scores),
       "score_weighted sizes");
  return launched();
}

hipError_t launch_select_topk(int32_t*, int64_t kept_ld, int32_t*, const float*, int64_t ld,
                              int64_t num_lists, int32_t n, int32_t K, int32_t prot, int32_t,
                              int32_t, const int32_t*, hipStream_t) {
  need(num_lists >= 0 && num_lists <= 2147483647 && prot >= 0 && K >= prot && n >= K && ld >= n &&
           kept_ld >= K,
       "select_topk sizes");
  return launched();
}

hipError_t launch_reduce_max_heads(float*, int64_t out_ld, const float*, int64_t ld,
                                   int64_t num_groups, int32_t H, int32_t n, hipStream_t) {
  need(num_groups >= 0 && H >= 1 && n >= 0 && ld >= n && out_ld >= n, "reduce_max_heads sizes");
  return launched();
}

size_t select_global_workspace_bytes(int64_t num_lists, int32_t n, int32_t prot) {
  need(num_lists >= 0 && n >= prot && prot >= 0, "workspace sizes");
  return 4096 + (size_t)num_lists * 64;
}

hipError_t launch_select_global(int32_t*, int64_t kept_ld, int32_t*, const float*, int64_t ld,
                                int64_t num_lists, int32_t n, int32_t prot, int64_t budget,
                                void* workspace, hipStream_t, bool) {
  need(num_lists >= 0 && (int64_t)num_lists * n <= 2147483647 && prot >= 0 && prot <= n &&
           ld >= n && kept_ld >= n && budget >= 0 && budget <= num_lists * (int64_t)(n - prot) &&
           workspace,
       "select_global sizes");
  return launched();
}

bool compact_orders_pages(const StoreView&, const StoreView& dst, int32_t, int32_t, int32_t K,
                          int64_t num_groups) {
  return dst.paged && K > 0 && num_groups > 0;
}

size_t compact_order_workspace_bytes(const StoreView& dst) {
  need(dst.capacity >= 0, "order workspace sizes");
  return (size_t)(dst.capacity * 4 + 256 + 255) / 256 * 256;
}

hipError_t launch_copy_pages(const void* k_src, const void* v_src, int64_t src_pages,
                             const int32_t* src_ids, void* k_dst, void* v_dst, int64_t dst_pages,
                             const int32_t* dst_ids, int64_t count, int64_t page_bytes,
                             uint32_t*, hipStream_t) {
  need(count > 0 && src_pages >= 0 && dst_pages >= 0 && page_bytes > 0 && page_bytes % 16 == 0 &&
           k_src && v_src && k_dst && v_dst && src_ids && dst_ids,
       "copy_pages sizes");
  return launched();
}

hipError_t select_global_scratch(void** ptr, size_t* bytes) {
  alignas(256) static unsigned char stand_in[256];  // a stand-in address, never dereferenced
  *ptr = &stand_in;
  *bytes = 1086208;
  return hipSuccess;
}

hipError_t launch_select_global_init(int32_t*, int64_t, int32_t*, int64_t num_lists, int32_t n,
                                     int32_t prot, int64_t budget, void* workspace, hipStream_t) {
  need(num_lists >= 0 && prot >= 0 && prot <= n && budget >= 0 && workspace, "init sizes");
  return launched();
}

uint32_t* select_global_first_level_bins(int64_t, int32_t, int32_t, int64_t, void* workspace) {
  return static_cast<uint32_t*>(workspace);
}

hipError_t launch_compact(const StoreView& src, const void*, const void*, const StoreView& dst,
                          void*, void*, int32_t D, int32_t H, const int32_t*, int64_t kept_ld,
                          const int32_t*, int32_t K, int64_t num_groups, int32_t ipg, uint32_t*,
                          hipStream_t, void*) {
  need(D > 0 && D % 8 == 0 && H >= 1 && (ipg == 1 || ipg == H) && K >= 0 && kept_ld >= K &&
           num_groups >= 0 && num_groups * (int64_t)H <= 2147483647 && K <= dst.max_rows &&
           src.max_rows >= 0,
       "compact sizes");
  return launched();
}

hipError_t launch_score_keydiff(float*, int64_t ld, const StoreView& keys, const void*, int32_t D,
                                int32_t H, int64_t num_lists, int32_t n, int32_t prot,
                                hipStream_t) {
  need(D >= 8 && D <= 512 && (D & (D - 1)) == 0 && H >= 1 && num_lists >= 0 &&
           num_lists <= 2147483647 && n >= 0 && prot >= 0 && prot <= n && ld >= n &&
           n <= keys.max_rows,
       "keydiff sizes");
  return launched();
}

hipError_t launch_compact_inplace(const StoreView& st, void*, void*, int32_t D, int32_t H,
                                  const int32_t*, int64_t kept_ld, const int32_t*, int32_t K,
                                  int32_t n, int64_t num_groups, int32_t ipg, int32_t*, uint32_t*,
                                  uint32_t*, hipStream_t) {
  need(D > 0 && H >= 1 && (ipg == 1 || ipg == H) && K >= 0 && K <= n && kept_ld >= K &&
           n <= st.max_rows && num_groups >= 0 && num_groups * (int64_t)H <= 2147483647,
       "compact_inplace sizes");
  return launched();
}

hipError_t launch_draw_select(int32_t*, int64_t kept_ld, int64_t num_lists, int32_t L, int32_t H,
                              int32_t n, int32_t K, int32_t prot, uint64_t, uint32_t, bool,
                              hipStream_t) {
  need(num_lists >= 0 && num_lists <= 2147483647 && L >= 1 && H >= 1 && prot >= 0 && K >= prot &&
           n >= K && kept_ld >= K,
       "draw_select sizes");
  return launched();
}

size_t evict_pages_lds_bytes(int32_t P, int32_t pp, int32_t Kp) {
  need(P >= 0 && pp >= 0 && Kp >= 0, "page counts");
  return (size_t)(P + pp + Kp) * 8;
}

hipError_t launch_evict_pages(int32_t* page_table, int64_t pt_ld, int32_t page_size,
                              int64_t num_groups, int32_t L, int32_t n, int32_t K, int32_t prot,
                              uint64_t, uint32_t, int32_t*, int64_t, int32_t*, uint32_t*,
                              hipStream_t) {
  need(page_size >= 1 && num_groups >= 0 && num_groups <= 2147483647 && L >= 1 && prot >= 0 &&
           K >= prot && n >= K && pt_ld >= n / page_size && (num_groups == 0 || page_table),
       "evict_pages sizes");
  return launched();
}

hipError_t launch_evict_random_inplace(const StoreView& st, void*, void*, int32_t D, int32_t H,
                                       int64_t num_groups, int32_t L, int32_t n, int32_t K,
                                       int32_t prot, uint64_t, uint32_t, bool, int32_t*,
                                       int64_t, int32_t*, uint32_t*, uint32_t*, hipStream_t) {
  need(D > 0 && H >= 1 && num_groups >= 0 && num_groups * (int64_t)H <= 2147483647 && L >= 1 &&
           prot >= 0 && K >= prot && n >= K && n <= st.max_rows &&
           (int64_t)(n - prot) + K <= kMaxFusedEntries,
       "evict_random_inplace sizes");
  return launched();
}

}  // namespace kvevict
