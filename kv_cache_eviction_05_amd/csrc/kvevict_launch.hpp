// Host-side launch interfaces between the C ABI (api.cpp) and the kernels.
// Every launcher assumes its arguments were validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvevict {

// A launch holds fewer than 2^32 work-items in each grid dimension: the most workgroups of
// `threads` threads that one dimension takes.  A launcher whose grid would not fit returns
// hipErrorInvalidConfiguration before it enqueues anything.
constexpr int64_t max_workgroups(int threads) { return 0xffffffffLL / threads; }
// Workgroup sizes of launches whose grid grows with the lists or tokens of a call (the
// kernels assert that they match), for callers that check a whole call before its first launch.
constexpr int kGlobalThreads = 1024;   // global top-B: one workgroup per list (init) or item
constexpr int kWeightedThreads = 512;  // weighted scores: one workgroup per tile of tokens
constexpr int kWeightedTile = 64;      // tokens per tile

hipError_t launch_score_random(float* scores, int64_t ld, int64_t num_lists, int32_t L, int32_t H,
                               int32_t n, int32_t prot, uint64_t seed, uint32_t round,
                               bool shared_draw, hipStream_t stream);

constexpr int kMaxWeightedLayers = 64;
struct WindowTable {
  int32_t begin[kMaxWeightedLayers];
  int32_t count[kMaxWeightedLayers];
};

// First level of the global top-B: 2048 bins of rank key bits [21, 32).
constexpr int kGlobalFirstLevelBins = 2048;

// hist0 (optional): the first-level bins of a global top-B over these scores
// (select_global_first_level_bins); every launch adds its scores of
// candidates t >= prot to them.
hipError_t launch_score_weighted(float* scores, int64_t ld, const float* beta, const float* vnorm,
                                 int64_t sg, int64_t st, int64_t sj, const float* w,
                                 int32_t w_slots, const WindowTable& win, int32_t L, int32_t H,
                                 int32_t Hg, int32_t n, int32_t prot, hipStream_t stream,
                                 uint32_t* hist0 = nullptr);

constexpr int kMaxBudgetLayers = 64;

// Per-head top-K: every list keeps K (layer_kk == nullptr) or, with per-layer
// budgets, prot + layer_kk[(list / H) % L]; kept_count (optional) receives the count.
hipError_t launch_select_topk(int32_t* kept_idx, int64_t kept_ld, int32_t* kept_count,
                              const float* scores, int64_t ld, int64_t num_lists, int32_t n,
                              int32_t K, int32_t prot, int32_t L, int32_t H,
                              const int32_t* layer_kk, hipStream_t stream);

hipError_t launch_reduce_max_heads(float* out, int64_t out_ld, const float* scores, int64_t ld,
                                   int64_t num_groups, int32_t H, int32_t n, hipStream_t stream);

size_t select_global_workspace_bytes(int64_t num_lists, int32_t n, int32_t prot);

// The current device's copy of the select's static scratch array (looked up on
// the first call on each device) and its size in bytes.  No allocation.
hipError_t select_global_scratch(void** ptr, size_t* bytes);

// The whole global top-B (first_level_done = false), or, after
// launch_select_global_init and a producer that filled the first-level bins,
// the rest of it (first_level_done = true).
hipError_t launch_select_global(int32_t* kept_idx, int64_t kept_ld, int32_t* kept_count,
                                const float* scores, int64_t ld, int64_t num_lists, int32_t n,
                                int32_t prot, int64_t budget, void* workspace, hipStream_t stream,
                                bool first_level_done = false);
// Prompt indices, prompt counts and the cleared workspace (before any producer adds bins).
hipError_t launch_select_global_init(int32_t* kept_idx, int64_t kept_ld, int32_t* kept_count,
                                     int64_t num_lists, int32_t n, int32_t prot, int64_t budget,
                                     void* workspace, hipStream_t stream);
// The 2048 first-level bins (rank key bits [21, 32) of the candidates) inside
// the workspace, or nullptr when the budget keeps nothing or everything.
uint32_t* select_global_first_level_bins(int64_t num_lists, int32_t n, int32_t prot,
                                         int64_t budget, void* workspace);

// Whole pages of K and V from src_ids to dst_ids (page_bytes a multiple of 16).
hipError_t launch_copy_pages(const void* k_src, const void* v_src, int64_t src_pages,
                             const int32_t* src_ids, void* k_dst, void* v_dst, int64_t dst_pages,
                             const int32_t* dst_ids, int64_t count, int64_t page_bytes,
                             uint32_t* errors, hipStream_t stream);

// One K/V store as the compaction kernels see it (units: 16-byte vectors).
struct StoreView {
  int32_t paged;
  int32_t page_shift;      // log2(page_size) when paged
  int64_t capacity;        // rows per list (contig) or pages in the pool (paged)
  int64_t list_stride_v;   // contig: 16-byte vectors between lists
  const int32_t* page_table;
  int64_t pt_ld;
  int64_t max_rows;        // rows addressable per list
};

hipError_t launch_compact(const StoreView& src, const void* k_src, const void* v_src,
                          const StoreView& dst, void* k_dst, void* v_dst, int32_t D, int32_t H,
                          const int32_t* kept_idx, int64_t kept_ld, const int32_t* kept_count,
                          int32_t K, int64_t num_groups, int32_t ipg, uint32_t* errors,
                          hipStream_t stream, void* order_ws = nullptr);

// The paged destination-ordered gather: whether it applies (a paged
// destination, one destination page per work item of the group kernel), and
// the workspace it takes (the pool's pages as int32 slots, and a flag).
bool compact_orders_pages(const StoreView& src, const StoreView& dst, int32_t D, int32_t H,
                          int32_t K, int64_t num_groups);
size_t compact_order_workspace_bytes(const StoreView& dst);

// KeyDiff scores of num_lists lists of n keys (D a power of two in [8, 512]).
hipError_t launch_score_keydiff(float* scores, int64_t ld, const StoreView& keys, const void* k,
                                int32_t D, int32_t H, int64_t num_lists, int32_t n, int32_t prot,
                                hipStream_t stream);

// In-place compaction of num_groups groups of one store (rows move to the
// front); paged: the tail pages beyond ceil(count_max / page_size) of the
// first n rows are appended to freed at atomicAdd(freed_count, ...).
hipError_t launch_compact_inplace(const StoreView& st, void* k, void* v, int32_t D, int32_t H,
                                  const int32_t* kept_idx, int64_t kept_ld,
                                  const int32_t* kept_count, int32_t K, int32_t n,
                                  int64_t num_groups, int32_t ipg, int32_t* freed,
                                  uint32_t* freed_count, uint32_t* errors, hipStream_t stream);

// Random draw + pin + top-K per list, the keys drawn in LDS (no score buffer).
hipError_t launch_draw_select(int32_t* kept_idx, int64_t kept_ld, int64_t num_lists, int32_t L,
                              int32_t H, int32_t n, int32_t K, int32_t prot, uint64_t seed,
                              uint32_t round, bool shared_draw, hipStream_t stream);

// Page-granular draw + pin + top pages, applied as page-table edits; the
// draws, old table row and kept pages of a group live in LDS.
size_t evict_pages_lds_bytes(int32_t P, int32_t pp, int32_t Kp);
hipError_t launch_evict_pages(int32_t* page_table, int64_t pt_ld, int32_t page_size,
                              int64_t num_groups, int32_t L, int32_t n, int32_t K, int32_t prot,
                              uint64_t seed, uint32_t round, int32_t* kept_pages, int64_t kept_ld,
                              int32_t* freed, uint32_t* freed_count, hipStream_t stream);

// Random draw + pin + top-K + in-place compaction of every (group, head) in
// one launch; (n - prot) + K keys and indices live in LDS.
constexpr int32_t kMaxFusedEntries = 15360;
hipError_t launch_evict_random_inplace(const StoreView& st, void* k, void* v, int32_t D,
                                       int32_t H, int64_t num_groups, int32_t L, int32_t n,
                                       int32_t K, int32_t prot, uint64_t seed, uint32_t round,
                                       bool shared_draw, int32_t* kept_idx, int64_t kept_ld,
                                       int32_t* freed, uint32_t* freed_count, uint32_t* errors,
                                       hipStream_t stream);

}  // namespace kvevict
