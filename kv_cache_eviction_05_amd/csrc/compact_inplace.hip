// In-place chronological compaction with a free-page list (GateSight Sec. 4.3
// and Appendix G: each layer moves the entries it keeps to the front of its
// own pages and the freed tail blocks return to the pool; "Random Attention"
// blog summary: per-KV-head physical eviction with chronological compaction).
//
//   row (g, h, j) <- row (g, h, idx[j])   for j < count, K and V, in place;
//   paged: pages ceil(count_max / page_size) .. ceil(n / page_size) - 1 of
//   group g are appended to the free list.
//
// Kept indices are strictly increasing, so idx[j] >= j: a row only moves
// towards the front, and the unchanged prefix (idx[j] == j: the prompt and the
// rows before the first eviction) is never touched.  Heads own disjoint
// memory in both layouts, so one workgroup per (group, head), head-major, walks
// that head's destination rows in increasing chunks.  Within a chunk a source row may also
// be a destination of the same chunk, so every thread waits for its loads
// before a workgroup barrier and only then stores; a later chunk reads only
// rows at or beyond its own first destination row, which no earlier chunk
// writes.  The walk is software-pipelined three deep: while the rows of chunk
// q are loaded, the page ids of chunk q+1 and the kept indices of chunk q+2
// are fetched, so each chunk waits on one memory latency, not four.
// The first moved row of the list is found with one round of 256 samples and
// a scan of the gap before the first mismatching sample.
#include "kvevict_device.hpp"
#include "kvevict_launch.hpp"

namespace kvevict {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kVecs = 8;  // 16-byte vectors of K (and of V) per thread per chunk
constexpr int32_t kChunk = kThreads * kVecs;

typedef uint32_t vec4u __attribute__((ext_vector_type(4)));

struct InplaceArgs {
  StoreView st;
  vec4u* k;
  vec4u* v;
  const int32_t* kept_idx;
  int64_t kept_ld;
  const int32_t* kept_count;
  int32_t K, H, ipg, vpr, n;
  int32_t* freed;
  uint32_t* freed_count;
  uint32_t* errors;
};

__device__ __forceinline__ int32_t count_of(const InplaceArgs& a, int64_t idx_list) {
  if (!a.kept_count) return a.K;
  const int32_t c = a.kept_count[idx_list];
  return c < 0 ? 0 : (c > a.K ? a.K : c);
}

// Smallest thread index whose flag is set, or kThreads (whole workgroup).
__device__ __forceinline__ int32_t block_first(bool hit, int32_t* s_min) {
  const int wave = threadIdx.x / kWave;
  const uint64_t b = __ballot(hit);
  if (lane_id() == 0) s_min[wave] = b ? wave * kWave + (int32_t)__builtin_ctzll(b) : kThreads;
  __syncthreads();
  int32_t r = s_min[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = min(r, s_min[w]);
  __syncthreads();
  return r;
}

// Smallest j < c with idx[j] != j, or c if the list keeps its prefix whole.
// idx[j] != j is false up to the first moved row and true from there on.
__device__ int32_t first_moved(const int32_t* __restrict__ idx, int32_t c, int32_t* s_min) {
  if (c <= 0) return c;
  const int32_t tid = threadIdx.x;
  const int32_t step = (c + kThreads - 1) / kThreads;
  const int32_t s = tid * step;
  const int32_t q = block_first(s < c && idx[s] != s, s_min);
  int32_t lo, hi;  // the first moved row lies in [lo, hi], or is c if none
  if (q < kThreads) {
    lo = q == 0 ? 0 : (q - 1) * step + 1;
    hi = q * step;
  } else {
    lo = ((c - 1) / step) * step + 1;
    hi = c - 1;
  }
  for (int32_t b = lo; b <= hi; b += kThreads) {
    const int32_t j = b + tid;
    const int32_t r = block_first(j <= hi && idx[j] != j, s_min);
    if (r < kThreads) return b + r;
  }
  return c;
}

template <bool kPaged>
__global__ __launch_bounds__(kThreads) void compact_inplace_kernel(InplaceArgs a) {
  __shared__ int32_t s_min[kWaves];
  // consecutive workgroups take one head of consecutive groups (head-major), so the
  // workgroups in flight do not all move rows of the same groups' pages at once
  // (same-process A/B against group-major: paged 3.917 -> 3.856 ms, the 30-round
  // shape in one round 15.86 -> 15.62 ms)
  const int32_t H = a.H;
  const int64_t G = gridDim.x / H;
  const int32_t h = (int32_t)(blockIdx.x / G);
  const int64_t g = blockIdx.x - (int64_t)h * G;
  const int32_t tid = threadIdx.x;
  const int64_t il = g * a.ipg + (a.ipg == 1 ? 0 : h);
  const int32_t* __restrict__ idx = a.kept_idx + il * a.kept_ld;
  const int32_t c = count_of(a, il);
  const int32_t first = first_moved(idx, c, s_min);
  const int32_t vpr = a.vpr;
  const int32_t E = (c - first) * vpr;  // vectors of the rows [first, c)
  const int32_t nq = (E + kChunk - 1) / kChunk;
  const int32_t* __restrict__ pt = kPaged ? a.st.page_table + g * a.st.pt_ld : nullptr;
  const int32_t shift = a.st.page_shift, pmask = (1 << shift) - 1;
  const int64_t cap = a.st.capacity, max_rows = a.st.max_rows;
  const int64_t list_base = kPaged ? 0 : (g * H + h) * a.st.list_stride_v;
  vec4u* kb = a.k;
  vec4u* vb = a.v;

  // row j and kept index t of element u of chunk q (t == j: nothing to move)
  auto fetch_idx = [&](int32_t q, int32_t (&j)[kVecs], int32_t (&t)[kVecs]) {
#pragma unroll
    for (int u = 0; u < kVecs; ++u) {
      const int32_t e = q * kChunk + u * kThreads + tid;
      j[u] = -1;
      t[u] = -1;
      if (e < E) {
        j[u] = first + e / vpr;
        t[u] = idx[j[u]];
      }
    }
  };
  // page ids of the source and destination rows (paged only)
  auto fetch_pages = [&](const int32_t (&j)[kVecs], const int32_t (&t)[kVecs],
                         int32_t (&sp)[kVecs], int32_t (&dp)[kVecs]) {
#pragma unroll
    for (int u = 0; u < kVecs; ++u) {
      sp[u] = -1;
      dp[u] = -1;
      if (kPaged && t[u] != j[u]) {
        if (t[u] > j[u] && (int64_t)t[u] < max_rows) sp[u] = pt[t[u] >> shift];
        dp[u] = pt[j[u] >> shift];
      }
    }
  };

  int32_t j1[kVecs], t1[kVecs], sp1[kVecs], dp1[kVecs];  // chunk q: ready to move
  int32_t j2[kVecs], t2[kVecs];                          // chunk q + 1: indices known
  if (nq > 0) {
    fetch_idx(0, j1, t1);
    fetch_idx(1, j2, t2);
    fetch_pages(j1, t1, sp1, dp1);
  }
  for (int32_t q = 0; q < nq; ++q) {
    vec4u kr[kVecs], vr[kVecs];
    int64_t dof[kVecs];
#pragma unroll
    for (int u = 0; u < kVecs; ++u) {
      dof[u] = -1;
      const int32_t j = j1[u], t = t1[u];
      if (t == j) continue;  // unchanged row or no element
      const int32_t col = (q * kChunk + u * kThreads + tid) - (j - first) * vpr;
      int64_t so = -1, d = -1;
      if (t > j && (int64_t)t < max_rows) {
        if (kPaged) {
          if (sp1[u] >= 0 && sp1[u] < cap && dp1[u] >= 0 && dp1[u] < cap) {
            so = ((((int64_t)sp1[u] << shift) + (t & pmask)) * H + h) * vpr + col;
            d = ((((int64_t)dp1[u] << shift) + (j & pmask)) * H + h) * vpr + col;
          }
        } else {
          so = list_base + (int64_t)t * vpr + col;
          d = list_base + (int64_t)j * vpr + col;
        }
      }
      if (so >= 0) {
        kr[u] = __builtin_nontemporal_load(kb + so);
        vr[u] = __builtin_nontemporal_load(vb + so);
        dof[u] = d;
      } else if (col == 0 && a.errors) {
        atomicAdd(a.errors, 1u);  // index below its slot, out of range, or bad page
      }
    }
    int32_t sp2[kVecs], dp2[kVecs], j3[kVecs], t3[kVecs];
    fetch_pages(j2, t2, sp2, dp2);
    fetch_idx(q + 2, j3, t3);
    // every load of the chunk has returned before any thread stores
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kVecs; ++u) {
      if (dof[u] >= 0) {
        __builtin_nontemporal_store(kr[u], kb + dof[u]);
        __builtin_nontemporal_store(vr[u], vb + dof[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kVecs; ++u) {
      j1[u] = j2[u];
      t1[u] = t2[u];
      sp1[u] = sp2[u];
      dp1[u] = dp2[u];
      j2[u] = j3[u];
      t2[u] = t3[u];
    }
  }

  // --- paged: the first head's workgroup returns the group's tail pages -------
  if (kPaged && a.freed && h == 0) {
    __shared__ int32_t s_cmax;
    __shared__ uint32_t s_base;
    if (tid == 0) s_cmax = 0;
    __syncthreads();
    int32_t cm = 0;
    for (int32_t l = tid; l < a.ipg; l += kThreads) cm = max(cm, count_of(a, g * a.ipg + l));
    atomicMax(&s_cmax, cm);
    __syncthreads();
    const int32_t ps = 1 << shift;
    const int32_t keep = (s_cmax + ps - 1) / ps;
    const int32_t used = (a.n + ps - 1) / ps;
    const int32_t nfree = used > keep ? used - keep : 0;
    if (tid == 0 && nfree > 0) s_base = atomicAdd(a.freed_count, (uint32_t)nfree);
    __syncthreads();
    for (int32_t i = tid; i < nfree; i += kThreads) a.freed[s_base + i] = pt[keep + i];
  }
}

}  // namespace

hipError_t launch_compact_inplace(const StoreView& st, void* k, void* v, int32_t D, int32_t H,
                                  const int32_t* kept_idx, int64_t kept_ld,
                                  const int32_t* kept_count, int32_t K, int32_t n,
                                  int64_t num_groups, int32_t ipg, int32_t* freed,
                                  uint32_t* freed_count, uint32_t* errors, hipStream_t stream) {
  if (num_groups == 0 || H == 0) return hipSuccess;
  if (num_groups * H > 0x7fffffffLL || (int64_t)n * (D / 8) > (1LL << 30))
    return hipErrorInvalidValue;
  if (num_groups * H > max_workgroups(kThreads)) return hipErrorInvalidConfiguration;
  InplaceArgs a;
  a.st = st;
  a.k = static_cast<vec4u*>(k);
  a.v = static_cast<vec4u*>(v);
  a.kept_idx = kept_idx;
  a.kept_ld = kept_ld;
  a.kept_count = kept_count;
  a.K = K;
  a.H = H;
  a.ipg = ipg;
  a.vpr = D / 8;
  a.n = n;
  a.freed = freed;
  a.freed_count = freed_count;
  a.errors = errors;
  const dim3 grid((unsigned)(num_groups * H));
  if (st.paged)
    hipLaunchKernelGGL(compact_inplace_kernel<true>, grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(compact_inplace_kernel<false>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvevict
