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
// rows before the first eviction) is never touched.  One workgroup per group
// (all H heads, so paged writes are whole token rows) walks the destination
// rows in increasing chunks.  Within a chunk a source row may also be a
// destination of the same chunk, so every thread waits for its loads before a
// workgroup barrier and only then stores; a later chunk reads only rows at or
// beyond its own first destination row, which no earlier chunk writes.
// The first moved row of each index list is found with two rounds of 32
// samples before the walk starts.
#include "kvevict_device.hpp"
#include "kvevict_launch.hpp"

namespace kvevict {
namespace {

constexpr int kThreads = 256;
constexpr int kVecs = 4;     // 16-byte vectors of K (and of V) per thread per chunk
constexpr int kTeam = 32;    // threads searching one index list
constexpr int kMaxTeams = kThreads / kTeam;

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

// Vector offset of row t of (group g, head h), or -1 if t or its page id
// falls outside the store.
__device__ __forceinline__ int64_t row_offset(const StoreView& s, int64_t g, int32_t h, int32_t H,
                                              int32_t t, int32_t vpr) {
  if (t < 0 || (int64_t)t >= s.max_rows) return -1;
  if (!s.paged) return (g * H + h) * s.list_stride_v + (int64_t)t * vpr;
  const int32_t page = s.page_table[g * s.pt_ld + (t >> s.page_shift)];
  if (page < 0 || (int64_t)page >= s.capacity) return -1;
  const int64_t slot = ((int64_t)page << s.page_shift) + (t & ((1 << s.page_shift) - 1));
  return (slot * H + h) * vpr;
}

__device__ __forceinline__ int32_t count_of(const InplaceArgs& a, int64_t idx_list) {
  if (!a.kept_count) return a.K;
  const int32_t c = a.kept_count[idx_list];
  return c < 0 ? 0 : (c > a.K ? a.K : c);
}

// Bits of the calling thread's 32-lane team in a wave ballot.
__device__ __forceinline__ uint32_t team_bits(uint64_t ballot) {
  return (uint32_t)(ballot >> (32 * ((threadIdx.x % kWave) / kTeam)));
}

__global__ __launch_bounds__(kThreads) void compact_inplace_kernel(InplaceArgs a) {
  __shared__ int32_t s_first[kMaxTeams];
  __shared__ int32_t s_cmax[kMaxTeams];
  const int64_t g = blockIdx.x;
  const int tid = threadIdx.x;
  const int team = tid / kTeam, k = tid % kTeam;
  const int32_t nlists = a.ipg;  // index lists of the group

  // --- first moved row and largest count over the group's index lists -------
  int32_t first = 0x7fffffff, cmax = 0;
  for (int32_t l0 = 0; l0 < nlists; l0 += kMaxTeams) {
    const int32_t l = l0 + team;
    const bool have = l < nlists;  // uniform per team
    const int64_t il = g * a.ipg + (have ? l : 0);
    const int32_t c = have ? count_of(a, il) : 0;
    const int32_t* idx = a.kept_idx + il * a.kept_ld;
    // round 1: samples 0, step, 2*step, ... (idx[j] != j is false, then true)
    const int32_t step = c > 0 ? (c + kTeam - 1) / kTeam : 1;
    const int32_t s = k * step;
    uint32_t m = team_bits(__ballot(have && s < c && idx[s] != s));
    int32_t lo, hi;  // the first moved row lies in [lo, hi], or is c if none
    if (m) {
      const int32_t kk = __builtin_ctz(m);
      lo = kk == 0 ? 0 : (kk - 1) * step + 1;
      hi = kk * step;
    } else {  // after the last sample below c
      lo = c > 0 ? ((c - 1) / step) * step + 1 : 0;
      hi = c - 1;
    }
    // round 2: scan [lo, hi] in steps of 32
    int32_t f = c;
    for (int32_t b = lo; b <= hi && f == c; b += kTeam) {
      const int32_t j = b + k;
      m = team_bits(__ballot(have && j <= hi && j < c && idx[j] != j));
      if (m) f = b + __builtin_ctz(m);
    }
    if (have) {
      if (f < c) first = min(first, f);  // lists with nothing to move do not count
      cmax = max(cmax, c);
    }
  }
  if (k == 0) {
    s_first[team] = first;
    s_cmax[team] = cmax;
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < kMaxTeams; ++t) {
    first = min(first, s_first[t]);
    cmax = max(cmax, s_cmax[t]);
  }

  // --- move the rows [first, cmax) in chunks, loads before stores -------------
  const int32_t vpr = a.vpr, H = a.H;
  const int32_t tok_vecs = H * vpr;
  const int32_t rows = (kThreads * kVecs) / tok_vecs > 0 ? (kThreads * kVecs) / tok_vecs : 1;
  for (int32_t j0 = first; j0 < cmax; j0 += rows) {
    const int32_t nvec = min(rows, cmax - j0) * tok_vecs;
    vec4u kr[kVecs], vr[kVecs];
    int64_t dof[kVecs];
    for (int32_t base = 0; base < nvec; base += kThreads * kVecs) {
#pragma unroll
      for (int u = 0; u < kVecs; ++u) {
        const int32_t e = base + tid + u * kThreads;
        dof[u] = -1;
        if (e >= nvec) continue;
        const int32_t j = j0 + e / tok_vecs;
        const int32_t rem = e % tok_vecs;
        const int32_t h = rem / vpr, col = rem - h * vpr;
        const int64_t il = g * a.ipg + (a.ipg == 1 ? 0 : h);
        if (j >= count_of(a, il)) continue;
        const int32_t t = a.kept_idx[il * a.kept_ld + j];
        if (t == j) continue;  // unchanged row
        const int64_t so = t > j ? row_offset(a.st, g, h, H, t, vpr) : -1;
        const int64_t d = row_offset(a.st, g, h, H, j, vpr);
        if (so >= 0 && d >= 0) {
          kr[u] = __builtin_nontemporal_load(a.k + so + col);
          vr[u] = __builtin_nontemporal_load(a.v + so + col);
          dof[u] = d + col;
        } else if (col == 0 && a.errors) {
          atomicAdd(a.errors, 1u);  // index below its slot, out of range, or bad page
        }
      }
      // every load of the chunk has returned before any thread stores
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kVecs; ++u) {
        if (dof[u] >= 0) {
          __builtin_nontemporal_store(kr[u], a.k + dof[u]);
          __builtin_nontemporal_store(vr[u], a.v + dof[u]);
        }
      }
    }
  }

  // --- paged: return the tail pages of the group to the free list -------------
  if (a.st.paged && a.freed) {
    const int32_t ps = 1 << a.st.page_shift;
    const int32_t keep = (cmax + ps - 1) / ps;
    const int32_t used = (a.n + ps - 1) / ps;
    const int32_t nfree = used > keep ? used - keep : 0;
    __shared__ uint32_t s_base;
    if (tid == 0 && nfree > 0) s_base = atomicAdd(a.freed_count, (uint32_t)nfree);
    __syncthreads();
    for (int32_t i = tid; i < nfree; i += kThreads)
      a.freed[s_base + i] = a.st.page_table[g * a.st.pt_ld + keep + i];
  }
}

}  // namespace

hipError_t launch_compact_inplace(const StoreView& st, void* k, void* v, int32_t D, int32_t H,
                                  const int32_t* kept_idx, int64_t kept_ld,
                                  const int32_t* kept_count, int32_t K, int32_t n,
                                  int64_t num_groups, int32_t ipg, int32_t* freed,
                                  uint32_t* freed_count, uint32_t* errors, hipStream_t stream) {
  if (num_groups == 0) return hipSuccess;
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
  hipLaunchKernelGGL(compact_inplace_kernel, dim3((unsigned)num_groups), dim3(kThreads), 0, stream,
                     a);
  return hipGetLastError();
}

}  // namespace kvevict
