// Chronological compaction ("Random Attention" blog summary: per-KV-head
// physical eviction with chronological compaction; GateSight Sec. 4.3: each
// layer moves the entries it keeps to the front of its pages).
//
//   dst row (g, h, j) = src row (g, h, idx[j])   for j < count, K and V.
//
// Rows are moved as 16-byte vectors (VPR = D/8 vectors per row) with
// nontemporal loads and stores: every source row is read once and every
// destination row written once.  Two work decompositions, both measured on
// MI355X against plain copies of the same bytes:
//
//  * list kernel (both stores contiguous).  A work item is one (list, chunk of
//    rows), 16 KiB of K or of V; even workgroups move the K rows of an item
//    and odd ones the V rows.  Small items keep the set of workgroups in flight
//    on a compact address range: ~6.0-6.4 TB/s on 256-byte rows, against
//    5.2-5.3 TB/s for 128 KiB per-list chunks moving K and V together.  Each
//    thread fetches the kept indices of its four vectors first, then loads all
//    four, then stores them (same-process A/B against 8 KiB items without the
//    staging: +1.7% batch, +4% longgen, +3% global).
//  * group kernel (either store paged).  A work item is 32 KiB of K and of V
//    destination rows of one group over all H heads (one whole 16-token page
//    at D = 128, H = 8), K and V in the same thread, so a workgroup writes a
//    whole destination page and reads the nearby source tokens of every head.
//    Each thread fetches all its indices and page ids, then loads all its
//    rows, then stores them, so the dependent latencies overlap.  Measured
//    against 8 KiB items (four tokens): +2.5%; against per-head chunks: ~+20%.
//
// Work items are visited by a grid-stride loop, so a one-shot grid (one item
// per workgroup) and a grid capped below 2^32 work-items run the same code.
// With per-list counts (kept_count, bounded only by K), a list is served by a
// team of workgroups walking strided chunks up to its own count, so lists far
// shorter than K do not launch mostly empty workgroups.
//
// Every indirect index (kept index, page id) is checked against its store
// before it is used; a row that fails is skipped and counted in *errors.
#include <algorithm>

#include "kvevict_device.hpp"
#include "kvevict_launch.hpp"

namespace kvevict {
namespace {

constexpr int kListThreads = 256;
constexpr int kListVecs = 1024;   // 16-byte vectors of K (or of V) per list item: 16 KiB
constexpr int kGroupThreads = 256;
constexpr int kGroupVecs = 2048;  // vectors of K and of V per group item: 32 KiB each
constexpr int kXcds = 8;  // accelerator dies of an MI355X, each with its own L2
constexpr int64_t kMaxGrid = 1 << 23;  // workgroups per launch (a multiple of kXcds): 256-thread groups stay below 2^31 work-items
static_assert(kMaxGrid % kXcds == 0, "the ordered walk keeps each workgroup on one XCD");
static_assert(kMaxGrid * kListThreads < (1LL << 32) && kMaxGrid * kGroupThreads < (1LL << 32),
              "a launch stays below 2^32 work-items");
// Chunks a workgroup pair walks at most with per-list counts (same-process A/B on
// 64 lists of 32768 rows keeping 600-22000 each: 4 beats 8 by 4%, 2 and 16 lose).
constexpr int32_t kVariableChunksPerPair = 4;

typedef uint32_t vec4u __attribute__((ext_vector_type(4)));

struct CompactArgs {
  StoreView src, dst;
  const vec4u* k_src;
  const vec4u* v_src;
  vec4u* k_dst;
  vec4u* v_dst;
  const int32_t* kept_idx;
  int64_t kept_ld;
  const int32_t* kept_count;
  int32_t K, H, ipg;
  int32_t rows_per_item;  // rows of one work item
  int32_t chunks;         // group kernel: items per group
  int32_t team;           // list kernel: workgroup pairs per list
  int64_t items;          // group items, or list workgroup pairs
  int32_t vpr;                    // 16-byte vectors per row
  uint32_t* errors;
  // group kernel, destination-ordered walk: slot s of the pool holds the item
  // whose destination page is s (or -1); *order_bad is set when some item's
  // page is outside the pool or shared, and the walk is then in item order
  const int32_t* order;
  const uint32_t* order_bad;
  int64_t order_len;
};

// Vector offset of row t of (group g, head h) in a store, or -1 if t or its
// page id falls outside the store.
__device__ __forceinline__ int64_t row_vec_offset(const StoreView& s, int64_t g, int32_t h,
                                                  int32_t H, int64_t list, int32_t t,
                                                  int32_t vpr) {
  if (t < 0 || (int64_t)t >= s.max_rows) return -1;
  if (!s.paged) return list * s.list_stride_v + (int64_t)t * vpr;
  const int32_t page = s.page_table[g * s.pt_ld + (t >> s.page_shift)];
  if (page < 0 || (int64_t)page >= s.capacity) return -1;
  const int64_t slot = ((int64_t)page << s.page_shift) + (t & ((1 << s.page_shift) - 1));
  return (slot * H + h) * vpr;
}

// Kept count of an index list, clamped to [0, K]; a count outside that range
// is reported once (by the first item of the list).
__device__ __forceinline__ int32_t list_count(const CompactArgs& a, int64_t idx_list,
                                              bool report) {
  if (!a.kept_count) return a.K;
  const int32_t c = a.kept_count[idx_list];
  if (c < 0 || c > a.K) {
    if (report && a.errors) atomicAdd(a.errors, 1u);
    return c < 0 ? 0 : a.K;
  }
  return c;
}

// VPR: vectors per row as a compile-time constant (0: a.vpr at run time).
// Workgroup pair p (K: even, V: odd) serves list p / team and walks the chunks
// p % team, p % team + team, ... below the list's count.
template <int VPR>
__global__ __launch_bounds__(kListThreads) void compact_list_kernel(CompactArgs a) {
  const int32_t vpr = VPR ? VPR : a.vpr;
  const bool is_v = blockIdx.x & 1;
  const vec4u* __restrict__ src = is_v ? a.v_src : a.k_src;
  vec4u* __restrict__ dst = is_v ? a.v_dst : a.k_dst;
  for (int64_t pair = blockIdx.x >> 1; pair < a.items; pair += gridDim.x >> 1) {
    const int64_t list = pair / a.team;
    const int32_t first_chunk = (int32_t)(pair - list * a.team);
    const int64_t g = list / a.H;
    const int32_t h = (int32_t)(list - g * a.H);
    const int64_t idx_list = g * a.ipg + (a.ipg == 1 ? 0 : h);
    const int32_t count = list_count(
        a, idx_list, first_chunk == 0 && !is_v && threadIdx.x == 0 && (a.ipg != 1 || h == 0));
    const int32_t* idx = a.kept_idx + idx_list * a.kept_ld;
    const int64_t step = (int64_t)a.team * a.rows_per_item;
    constexpr int kPer = (kListVecs + kListThreads - 1) / kListThreads;
    for (int64_t r0l = (int64_t)first_chunk * a.rows_per_item; r0l < count; r0l += step) {
      const int32_t r0 = (int32_t)r0l;
      const int32_t r1 = min(count, r0 + a.rows_per_item);
      const int32_t nvec = (r1 - r0) * vpr;
      for (int32_t base = 0; base < nvec; base += kPer * kListThreads) {
        int64_t so[kPer], dof[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
          so[u] = -1;
          const int32_t v = base + threadIdx.x + u * kListThreads;
          if (v >= nvec) continue;
          const int32_t row = r0 + v / vpr;
          const int32_t col = v % vpr;
          const int64_t s = row_vec_offset(a.src, g, h, a.H, list, idx[row], vpr);
          const int64_t d = row_vec_offset(a.dst, g, h, a.H, list, row, vpr);
          if (s >= 0 && d >= 0) {
            so[u] = s + col;
            dof[u] = d + col;
          } else if (col == 0 && !is_v && a.errors) {
            atomicAdd(a.errors, 1u);
          }
        }
        vec4u x[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u)
          if (so[u] >= 0) x[u] = __builtin_nontemporal_load(src + so[u]);
#pragma unroll
        for (int u = 0; u < kPer; ++u)
          if (so[u] >= 0) __builtin_nontemporal_store(x[u], dst + dof[u]);
      }
    }
  }
}

__global__ __launch_bounds__(kGroupThreads) void compact_group_kernel(CompactArgs a) {
  // Each thread moves at most kPer vectors of K and of V per item: all their
  // indices and page ids are fetched first, then all the rows are loaded, then
  // stored, so the three dependent memory latencies overlap across vectors.
  constexpr int kPer = (kGroupVecs + kGroupThreads - 1) / kGroupThreads;
  const int32_t vpr = a.vpr;
  const int32_t tok_vecs = a.H * vpr;  // vectors of one token row over all heads
  const vec4u* __restrict__ ks = a.k_src;
  const vec4u* __restrict__ vs = a.v_src;
  vec4u* __restrict__ kd = a.k_dst;
  vec4u* __restrict__ vd = a.v_dst;
  const bool ordered = a.order && *a.order_bad == 0u;
  // ordered: slots [0, kXcds * per_xcd) map one to one onto the pool's pages
  // (and past its end, where they idle); workgroup b runs on XCD b % 8
  // (round-robin dispatch, and the grid is a multiple of 8), so XCD x walks
  // the x-th eighth of the pool's pages in increasing order
  const int64_t per_xcd = (a.order_len + kXcds - 1) / kXcds;
  const int64_t slots = ordered ? per_xcd * kXcds : a.items;
  for (int64_t slot = blockIdx.x; slot < slots; slot += gridDim.x) {
    int64_t item = slot;
    if (ordered) {
      const int64_t s2 = (slot % kXcds) * per_xcd + slot / kXcds;
      if (s2 >= a.order_len) continue;
      item = a.order[s2];
      if (item < 0 || item >= a.items) continue;
    }
    const int64_t g = item / a.chunks;
    const int32_t chunk = (int32_t)(item - g * a.chunks);
    const int32_t r0 = chunk * a.rows_per_item;
    const int32_t r1 = min(a.K, r0 + a.rows_per_item);
    const int32_t nvec = (r1 - r0) * tok_vecs;
    for (int32_t base = 0; base < nvec; base += kPer * kGroupThreads) {
      int64_t so[kPer], dof[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        so[u] = -1;
        dof[u] = -1;
        const int32_t v = base + threadIdx.x + u * kGroupThreads;
        if (v >= nvec) continue;
        const int32_t row = r0 + v / tok_vecs;
        const int32_t rem = v % tok_vecs;
        const int32_t h = rem / vpr;
        const int32_t col = rem - h * vpr;
        const int64_t list = g * a.H + h;
        const int64_t idx_list = g * a.ipg + (a.ipg == 1 ? 0 : h);
        const bool first = (chunk == 0 && row == r0 && col == 0 && (a.ipg != 1 || h == 0));
        const int32_t count = list_count(a, idx_list, first);
        if (row >= count) continue;
        const int64_t s = row_vec_offset(a.src, g, h, a.H, list,
                                         a.kept_idx[idx_list * a.kept_ld + row], vpr);
        const int64_t d = row_vec_offset(a.dst, g, h, a.H, list, row, vpr);
        if (s >= 0 && d >= 0) {
          so[u] = s + col;
          dof[u] = d + col;
        } else if (col == 0 && a.errors) {
          atomicAdd(a.errors, 1u);
        }
      }
      vec4u x[kPer], y[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        if (so[u] >= 0) {
          x[u] = __builtin_nontemporal_load(ks + so[u]);
          y[u] = __builtin_nontemporal_load(vs + so[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        if (so[u] >= 0) {
          __builtin_nontemporal_store(x[u], kd + dof[u]);
          __builtin_nontemporal_store(y[u], vd + dof[u]);
        }
      }
    }
  }
}

// Destination-ordered walk of the group kernel: the pool's slots are cleared,
// then every item writes its index into the slot of its destination page (one
// whole page per item).  A page outside the pool, or one that two items name,
// sets *bad, and the gather then walks the items in their own order.
__global__ __launch_bounds__(256) void order_clear_kernel(int32_t* order, int64_t len,
                                                          uint32_t* bad) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < len; i += (int64_t)gridDim.x * 256)
    order[i] = -1;
  if (blockIdx.x == 0 && threadIdx.x == 0) *bad = 0u;
}

__global__ __launch_bounds__(256) void order_scatter_kernel(const int32_t* page_table, int64_t pt_ld,
                                                            int32_t page_shift, int32_t rows_per_item,
                                                            int32_t chunks, int64_t items,
                                                            int32_t* order, int64_t len,
                                                            uint32_t* bad) {
  const int64_t item = blockIdx.x * 256ll + threadIdx.x;
  if (item >= items) return;
  const int64_t g = item / chunks;
  const int32_t chunk = (int32_t)(item - g * chunks);
  const int32_t page = page_table[g * pt_ld + (((int64_t)chunk * rows_per_item) >> page_shift)];
  if (page < 0 || (int64_t)page >= len || atomicCAS(order + page, -1, (int32_t)item) != -1)
    atomicOr(bad, 1u);
}

struct Plan {
  bool group;
  int32_t rows_per_item, chunks, team;
  int64_t items, grid;
};

Plan plan_compact(const StoreView& src, const StoreView& dst, int32_t D, int32_t H, int32_t K,
                  int64_t num_groups, bool variable_counts) {
  Plan p{};
  const int32_t vpr = D / 8;
  p.group = src.paged || dst.paged;
  if (p.group) {
    const int32_t tok_vecs = H * vpr;
    p.rows_per_item = tok_vecs >= kGroupVecs ? 1 : kGroupVecs / tok_vecs;
    p.chunks = (K + p.rows_per_item - 1) / p.rows_per_item;
    p.items = num_groups * p.chunks;
    p.grid = p.items < kMaxGrid ? p.items : kMaxGrid;
  } else {
    p.rows_per_item = vpr >= kListVecs ? 1 : kListVecs / vpr;
    p.chunks = (K + p.rows_per_item - 1) / p.rows_per_item;
    // Uniform counts: one chunk per workgroup pair.  Variable counts (K only
    // bounds them): a quarter as many pairs, each walking up to four chunks,
    // so lists far below K do not leave most workgroups empty.
    p.team = variable_counts ? (p.chunks + kVariableChunksPerPair - 1) / kVariableChunksPerPair
                             : p.chunks;
    p.items = num_groups * H * p.team;
    const int64_t pairs = p.items < kMaxGrid / 2 ? p.items : kMaxGrid / 2;
    p.grid = 2 * pairs;  // even workgroups move K, odd ones V
  }
  return p;
}

}  // namespace

bool compact_orders_pages(const StoreView& src, const StoreView& dst, int32_t D, int32_t H,
                          int32_t K, int64_t num_groups) {
  if (!dst.paged || num_groups == 0 || K == 0) return false;
  const Plan p = plan_compact(src, dst, D, H, K, num_groups, false);
  // one destination page per item, and a pool not much larger than the pages written
  return p.group && p.rows_per_item == (1 << dst.page_shift) && dst.capacity <= 4 * p.items;
}

size_t compact_order_workspace_bytes(const StoreView& dst) {
  return (size_t)(dst.capacity * 4 + 256 + 255) / 256 * 256;
}

hipError_t launch_compact(const StoreView& src, const void* k_src, const void* v_src,
                          const StoreView& dst, void* k_dst, void* v_dst, int32_t D, int32_t H,
                          const int32_t* kept_idx, int64_t kept_ld, const int32_t* kept_count,
                          int32_t K, int64_t num_groups, int32_t ipg, uint32_t* errors,
                          hipStream_t stream, void* order_ws) {
  if (num_groups == 0 || K == 0) return hipSuccess;
  const Plan p = plan_compact(src, dst, D, H, K, num_groups, kept_count != nullptr);
  // one thread per item in the page-order scatter
  if ((p.items + 255) / 256 > max_workgroups(256)) return hipErrorInvalidConfiguration;
  CompactArgs a;
  a.src = src;
  a.dst = dst;
  a.k_src = static_cast<const vec4u*>(k_src);
  a.v_src = static_cast<const vec4u*>(v_src);
  a.k_dst = static_cast<vec4u*>(k_dst);
  a.v_dst = static_cast<vec4u*>(v_dst);
  a.kept_idx = kept_idx;
  a.kept_ld = kept_ld;
  a.kept_count = kept_count;
  a.K = K;
  a.H = H;
  a.ipg = ipg;
  a.rows_per_item = p.rows_per_item;
  a.chunks = p.chunks;
  a.team = p.team;
  a.items = p.items;
  a.vpr = D / 8;
  a.errors = errors;
  a.order = nullptr;
  a.order_bad = nullptr;
  a.order_len = 0;
  if (p.group) {
    int64_t grid = p.grid;
    if (order_ws && compact_orders_pages(src, dst, D, H, K, num_groups)) {
      int32_t* order = static_cast<int32_t*>(order_ws);
      const int64_t len = dst.capacity;
      uint32_t* bad = reinterpret_cast<uint32_t*>(static_cast<char*>(order_ws) +
                                                  (len * 4 + 255) / 256 * 256);
      const int64_t clear_grid = std::min<int64_t>((len + 255) / 256, 1 << 16);
      hipLaunchKernelGGL(order_clear_kernel, dim3((unsigned)std::max<int64_t>(clear_grid, 1)),
                         dim3(256), 0, stream, order, len, bad);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(order_scatter_kernel, dim3((unsigned)((p.items + 255) / 256)), dim3(256),
                         0, stream, dst.page_table, dst.pt_ld, dst.page_shift, p.rows_per_item,
                         p.chunks, p.items, order, len, bad);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      a.order = order;
      a.order_bad = bad;
      a.order_len = len;
      // enough workgroups for the larger of the walks (the pool's pages rounded up to a
      // multiple of the XCDs, or the items); kMaxGrid is a multiple of 8 as well
      const int64_t span = (len + kXcds - 1) / kXcds * kXcds;
      const int64_t slots = std::max<int64_t>(span, p.items);
      grid = slots < kMaxGrid ? slots : kMaxGrid;
    }
    hipLaunchKernelGGL(compact_group_kernel, dim3((unsigned)grid), dim3(kGroupThreads), 0,
                       stream, a);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)p.grid), block(kListThreads);
  switch (a.vpr) {
    case 16:
      hipLaunchKernelGGL(compact_list_kernel<16>, grid, block, 0, stream, a);
      break;
    case 32:
      hipLaunchKernelGGL(compact_list_kernel<32>, grid, block, 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL(compact_list_kernel<0>, grid, block, 0, stream, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace kvevict
