// One-kernel Random Attention round with in-place compaction ("Random
// Attention" blog summary, Algorithm 1: a random score per entry, the prompt
// pinned, top-K per KV head, keep set returned; engine paragraph: per-KV-head
// physical eviction with chronological compaction; GateSight Sec. 4.3 and
// Appendix G: kept entries move to the front of their own pages and the freed
// tail blocks return to the pool).
//
// One 256-thread workgroup per (group, head), head-major.  It draws the n - prot
// candidate scores of its list with the same Philox stream as the standalone
// scorer straight into LDS keys, selects the K - prot largest (ties to the
// lower position), writes the kept indices in increasing order into LDS (and,
// if asked, to the caller), and then moves its head's kept rows to the front
// in place exactly as the standalone in-place compaction does: chunks in
// increasing order, each one's loads complete before a workgroup barrier,
// then its stores.  Neither scores nor indices travel through HBM.  With a
// shared draw every head's workgroup draws the head-0 list of its group.
#include "kvevict_device.hpp"
#include "kvevict_launch.hpp"
#include "select_lds.hpp"

namespace kvevict {
namespace {

constexpr int kThreads = kSelectThreads;
constexpr int kWaves = kThreads / kWave;
constexpr int kVecs = 8;  // 16-byte vectors of K (and of V) per thread per chunk
constexpr int32_t kChunk = kThreads * kVecs;

typedef uint32_t vec4u __attribute__((ext_vector_type(4)));

struct FusedArgs {
  StoreView st;
  vec4u* k;
  vec4u* v;
  int32_t L, H, n, K, prot, vpr, shared_draw;
  uint64_t seed;
  uint32_t round;
  int32_t* kept_idx;  // optional
  int64_t kept_ld;
  int32_t* freed;
  uint32_t* freed_count;
  uint32_t* errors;
};

template <bool kPaged>
__global__ __launch_bounds__(kThreads) void evict_random_inplace_kernel(FusedArgs a) {
  extern __shared__ uint32_t s_dyn[];  // candidate keys [n - prot], then kept indices [K]
  __shared__ SelectShared<kThreads> sh;
  __shared__ int32_t s_min[kWaves];
  const int32_t H = a.H, n = a.n, K = a.K, prot = a.prot;
  // head-major, as the standalone in-place compaction (same-process A/B against
  // group-major: paged 3.895 -> 3.838 ms, the 30-round shape in one round 15.86 -> 15.57 ms)
  const int64_t G = gridDim.x / H;
  const int32_t h = (int32_t)(blockIdx.x / G);
  const int64_t g = blockIdx.x - (int64_t)h * G;
  const int32_t tid = threadIdx.x;
  const int32_t m = n - prot, kk = K - prot;
  uint32_t* s_keys = s_dyn;
  int32_t* s_kept = reinterpret_cast<int32_t*>(s_dyn + m);

  // --- score: the Philox draw of every candidate slot, as rank keys ----------
  const uint64_t request = (uint64_t)(g / a.L), layer = (uint64_t)(g % a.L);
  const uint64_t head = a.shared_draw ? 0u : (uint64_t)h;
  for (int32_t c = prot / 4 + tid; 4 * c < n; c += kThreads) {
    const Philox4x64 r =
        philox4x64_10((uint64_t)c, head, layer, (request << 32) | a.round, a.seed, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int32_t i = 4 * c + q;
      if (i >= prot && i < n) s_keys[i - prot] = draw_key(r.w[q]);
    }
  }
  for (int32_t j = tid; j < prot; j += kThreads) s_kept[j] = j;
  __syncthreads();

  // --- select and emit the kept indices in increasing order ------------------
  if (kk > 0) {
    auto key_at = [&](int32_t i) -> uint32_t { return s_keys[i]; };
    uint32_t thr = 0u, need_eq = 0xffffffffu;  // kk == m: keep every candidate
    if (kk < m) radix_select<24>(key_at, m, kk, sh, thr, need_eq);
    emit_kept(key_at, m, thr, need_eq, sh,
              [&](uint32_t slot, int32_t i) { s_kept[prot + slot] = prot + i; });
  }
  __syncthreads();
  if (a.kept_idx && (!a.shared_draw || h == 0)) {
    int32_t* out = a.kept_idx + (a.shared_draw ? g : g * H + h) * a.kept_ld;
    for (int32_t j = tid; j < K; j += kThreads) out[j] = s_kept[j];
  }

  // --- first moved row: the smallest j with kept[j] != j ----------------------
  int32_t first = K;
  for (int32_t b = prot; b < K; b += kThreads) {
    const int32_t j = b + tid;
    const uint64_t bal = __ballot(j < K && s_kept[j] != j);
    if (lane_id() == 0) s_min[tid / kWave] = bal ? (int32_t)__builtin_ctzll(bal) + (tid & ~(kWave - 1)) : kThreads;
    __syncthreads();
    int32_t r = s_min[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) r = min(r, s_min[w]);
    __syncthreads();
    if (r < kThreads) {
      first = b + r;
      break;
    }
  }

  // --- move the rows [first, K) of this head in place -------------------------
  const int32_t vpr = a.vpr;
  const int32_t E = (K - first) * vpr;
  const int32_t nq = (E + kChunk - 1) / kChunk;
  const int32_t* __restrict__ pt = kPaged ? a.st.page_table + g * a.st.pt_ld : nullptr;
  const int32_t shift = a.st.page_shift, pmask = (1 << shift) - 1;
  const int64_t cap = a.st.capacity;
  const int64_t list_base = kPaged ? 0 : (g * H + h) * a.st.list_stride_v;
  vec4u* kb = a.k;
  vec4u* vb = a.v;

  // row j and source row t of element u of chunk q (t == j: nothing to move)
  auto rows_of = [&](int32_t q, int32_t (&j)[kVecs], int32_t (&t)[kVecs]) {
#pragma unroll
    for (int u = 0; u < kVecs; ++u) {
      const int32_t e = q * kChunk + u * kThreads + tid;
      j[u] = -1;
      t[u] = -1;
      if (e < E) {
        j[u] = first + e / vpr;
        t[u] = s_kept[j[u]];
      }
    }
  };
  auto fetch_pages = [&](const int32_t (&j)[kVecs], const int32_t (&t)[kVecs],
                         int32_t (&sp)[kVecs], int32_t (&dp)[kVecs]) {
#pragma unroll
    for (int u = 0; u < kVecs; ++u) {
      sp[u] = -1;
      dp[u] = -1;
      if (kPaged && t[u] != j[u]) {
        sp[u] = pt[t[u] >> shift];
        dp[u] = pt[j[u] >> shift];
      }
    }
  };

  int32_t j1[kVecs], t1[kVecs], sp1[kVecs], dp1[kVecs];  // chunk q, page ids known
  if (nq > 0) {
    rows_of(0, j1, t1);
    fetch_pages(j1, t1, sp1, dp1);
  }
  for (int32_t q = 0; q < nq; ++q) {
    vec4u kr[kVecs], vr[kVecs];
    int64_t dof[kVecs];
#pragma unroll
    for (int u = 0; u < kVecs; ++u) {
      dof[u] = -1;
      const int32_t j = j1[u], t = t1[u];
      if (t == j) continue;
      const int32_t col = (q * kChunk + u * kThreads + tid) - (j - first) * vpr;
      int64_t so = -1, d = -1;
      if (kPaged) {
        if (sp1[u] >= 0 && sp1[u] < cap && dp1[u] >= 0 && dp1[u] < cap) {
          so = ((((int64_t)sp1[u] << shift) + (t & pmask)) * H + h) * vpr + col;
          d = ((((int64_t)dp1[u] << shift) + (j & pmask)) * H + h) * vpr + col;
        }
      } else {
        so = list_base + (int64_t)t * vpr + col;
        d = list_base + (int64_t)j * vpr + col;
      }
      if (so >= 0) {
        kr[u] = __builtin_nontemporal_load(kb + so);
        vr[u] = __builtin_nontemporal_load(vb + so);
        dof[u] = d;
      } else if (col == 0 && a.errors) {
        atomicAdd(a.errors, 1u);  // page id outside the pool
      }
    }
    int32_t j2[kVecs], t2[kVecs], sp2[kVecs], dp2[kVecs];
    rows_of(q + 1, j2, t2);
    fetch_pages(j2, t2, sp2, dp2);
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
    }
  }

  // --- paged: the first head's workgroup returns the group's tail pages -------
  if (kPaged && a.freed && h == 0) {
    __shared__ uint32_t s_base;
    const int32_t ps = 1 << shift;
    const int32_t keep = (K + ps - 1) / ps;
    const int32_t used = (n + ps - 1) / ps;
    const int32_t nfree = used > keep ? used - keep : 0;
    if (tid == 0 && nfree > 0) s_base = atomicAdd(a.freed_count, (uint32_t)nfree);
    __syncthreads();
    for (int32_t i = tid; i < nfree; i += kThreads) a.freed[s_base + i] = pt[keep + i];
  }
}

}  // namespace

size_t evict_fused_lds_bytes(int32_t n, int32_t K, int32_t prot) {
  return (size_t)((n - prot) + K) * sizeof(uint32_t);
}

hipError_t launch_evict_random_inplace(const StoreView& st, void* k, void* v, int32_t D,
                                       int32_t H, int64_t num_groups, int32_t L, int32_t n,
                                       int32_t K, int32_t prot, uint64_t seed, uint32_t round,
                                       bool shared_draw, int32_t* kept_idx, int64_t kept_ld,
                                       int32_t* freed, uint32_t* freed_count, uint32_t* errors,
                                       hipStream_t stream) {
  if (num_groups == 0 || H == 0) return hipSuccess;
  if (num_groups * H > max_workgroups(kThreads)) return hipErrorInvalidConfiguration;
  FusedArgs a;
  a.st = st;
  a.k = static_cast<vec4u*>(k);
  a.v = static_cast<vec4u*>(v);
  a.L = L;
  a.H = H;
  a.n = n;
  a.K = K;
  a.prot = prot;
  a.vpr = D / 8;
  a.shared_draw = shared_draw ? 1 : 0;
  a.seed = seed;
  a.round = round;
  a.kept_idx = kept_idx;
  a.kept_ld = kept_ld;
  a.freed = freed;
  a.freed_count = freed_count;
  a.errors = errors;
  const dim3 grid((unsigned)(num_groups * H));
  const size_t lds = evict_fused_lds_bytes(n, K, prot);
  if (st.paged)
    hipLaunchKernelGGL(evict_random_inplace_kernel<true>, grid, dim3(kThreads), lds, stream, a);
  else
    hipLaunchKernelGGL(evict_random_inplace_kernel<false>, grid, dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace kvevict
