// Chronological compaction ("Random Attention" blog summary: per-KV-head
// physical eviction with chronological compaction; GateSight Sec. 4.3: each
// layer moves the entries it keeps to the front of its pages).
//
//   dst row (g, h, j) = src row (g, h, idx[j])   for j < count, K and V.
//
// The work unit of a workgroup is (list = g*H + h, chunk of kRowsPerBlock
// destination rows).  Rows are moved as 16-byte vectors: VPR = D/8 lanes
// cover one row, so a wave moves 64/VPR whole rows per instruction with fully
// coalesced 16-byte accesses on both sides.  Each thread issues kUnroll
// K loads and kUnroll V loads before its stores, keeping 32 KiB per
// workgroup in flight to cover HBM latency.  Source rows are streamed once
// and destination rows written once, so both use nontemporal accesses.
//
// Every indirect index (kept index, page id) is checked against its store
// before it is used; a row that fails is skipped and counted in *errors.
#include "kvevict_device.hpp"
#include "kvevict_launch.hpp"

namespace kvevict {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int kVecsPerBlock = 8192;  // 128 KiB of K (+ the same of V) per workgroup

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
  int32_t rows_per_block, chunks_per_list;
  int32_t vpr;  // runtime vectors per row (generic instantiation)
  uint32_t* errors;
};

// Vector offset of row t of (group g, head h) in a store, or -1 if t or its
// page id falls outside the store.
template <int VPR>
__device__ __forceinline__ int64_t row_vec_offset(const StoreView& s, int64_t g, int32_t h,
                                                  int32_t H, int64_t list, int32_t t, int vpr) {
  const int64_t vrow = VPR ? VPR : vpr;
  if (t < 0 || (int64_t)t >= s.max_rows) return -1;
  if (!s.paged) return list * s.list_stride_v + (int64_t)t * vrow;
  const int32_t page = s.page_table[g * s.pt_ld + (t >> s.page_shift)];
  if (page < 0 || (int64_t)page >= s.capacity) return -1;
  const int64_t slot = ((int64_t)page << s.page_shift) + (t & ((1 << s.page_shift) - 1));
  return (slot * H + h) * vrow;
}

template <int VPR>
__global__ __launch_bounds__(kThreads) void compact_kernel(CompactArgs a) {
  const int vpr = VPR ? VPR : a.vpr;
  const int64_t list = blockIdx.x / a.chunks_per_list;
  const int32_t chunk = blockIdx.x % a.chunks_per_list;
  const int64_t g = list / a.H;
  const int32_t h = (int32_t)(list % a.H);
  const int64_t idx_list = g * a.ipg + (a.ipg == 1 ? 0 : h);

  int32_t count = a.K;
  if (a.kept_count) {
    count = a.kept_count[idx_list];
    if (count < 0 || count > a.K) {
      if (chunk == 0 && threadIdx.x == 0 && a.errors) atomicAdd(a.errors, 1u);
      count = count < 0 ? 0 : a.K;
    }
  }
  const int32_t r0 = chunk * a.rows_per_block;
  if (r0 >= count) return;
  const int32_t r1 = min(count, r0 + a.rows_per_block);
  const int32_t* idx = a.kept_idx + idx_list * a.kept_ld;
  const int32_t nvec = (r1 - r0) * vpr;

  for (int32_t v0 = threadIdx.x; v0 < nvec; v0 += kThreads * kUnroll) {
    vec4u kr[kUnroll], vr[kUnroll];
    int64_t doff[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int32_t v = v0 + u * kThreads;
      doff[u] = -1;
      if (v < nvec) {
        const int32_t row = r0 + v / vpr;
        const int32_t col = v % vpr;
        const int32_t t = idx[row];
        const int64_t so = row_vec_offset<VPR>(a.src, g, h, a.H, list, t, vpr);
        const int64_t dof = row_vec_offset<VPR>(a.dst, g, h, a.H, list, row, vpr);
        if (so >= 0 && dof >= 0) {
          kr[u] = __builtin_nontemporal_load(a.k_src + so + col);
          vr[u] = __builtin_nontemporal_load(a.v_src + so + col);
          doff[u] = dof + col;
        } else if (col == 0 && a.errors) {
          atomicAdd(a.errors, 1u);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (doff[u] >= 0) {
        __builtin_nontemporal_store(kr[u], a.k_dst + doff[u]);
        __builtin_nontemporal_store(vr[u], a.v_dst + doff[u]);
      }
    }
  }
}

int32_t rows_per_block(int32_t D, int32_t K) {
  int32_t rows = kVecsPerBlock / (D / 8);
  if (rows < 1) rows = 1;
  if (rows > K) rows = K;
  return rows;
}

}  // namespace

int64_t compact_workgroups(int32_t D, int32_t K, int64_t lists) {
  if (K <= 0) return 0;
  const int32_t rows = rows_per_block(D, K);
  return lists * ((K + rows - 1) / rows);
}

hipError_t launch_compact(const StoreView& src, const void* k_src, const void* v_src,
                          const StoreView& dst, void* k_dst, void* v_dst, int32_t D, int32_t H,
                          const int32_t* kept_idx, int64_t kept_ld, const int32_t* kept_count,
                          int32_t K, int64_t num_groups, int32_t ipg, uint32_t* errors,
                          hipStream_t stream) {
  if (num_groups == 0 || K == 0) return hipSuccess;
  const int32_t vpr = D / 8;
  const int32_t rows = rows_per_block(D, K);
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
  a.rows_per_block = rows;
  a.chunks_per_list = (K + rows - 1) / rows;
  a.vpr = vpr;
  a.errors = errors;
  const int64_t blocks = num_groups * H * a.chunks_per_list;
  const dim3 grid((unsigned)blocks), block(kThreads);
  switch (vpr) {
    case 8:
      hipLaunchKernelGGL(compact_kernel<8>, grid, block, 0, stream, a);
      break;
    case 16:
      hipLaunchKernelGGL(compact_kernel<16>, grid, block, 0, stream, a);
      break;
    case 32:
      hipLaunchKernelGGL(compact_kernel<32>, grid, block, 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL(compact_kernel<0>, grid, block, 0, stream, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace kvevict
