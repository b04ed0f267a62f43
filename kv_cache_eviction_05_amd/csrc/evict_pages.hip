// Page-granular Random Attention eviction as page-table edits ("Random
// Attention" blog summary, Algorithm 1 applied to the blocks of a paged cache:
// a random score per block, the prompt pinned, the top blocks kept; GateSight
// Sec. 4.3: one block table per layer over a shared pool, freed blocks return
// to the pool).
//
// A page holds page_size token slots of every KV head, so one list per
// (request, layer): page b scores the shared (head-0) draw of its first slot
// b*page_size.  Pages holding a prompt slot are kept; of the others the
// K/page_size - ceil(prot/page_size) largest, ties to the lower page.  The
// kept pages' physical ids move to the front of the group's table row in page
// order, the rest of the row's first n/page_size entries become -1, and the
// evicted ids are appended to the free list in page order.  No K/V byte moves.
//
// One 256-thread workgroup per group: page draws and the old table row go to
// LDS, the radix select and chronological emit of select_lds.hpp pick the kept
// pages, then the row is rewritten and the free list written from LDS.
#include "kvevict_device.hpp"
#include "kvevict_launch.hpp"
#include "select_lds.hpp"

namespace kvevict {
namespace {

constexpr int kThreads = kSelectThreads;

struct PagesArgs {
  int32_t* pt;
  int64_t pt_ld;
  int32_t ps, P, pp, Kp, L;
  uint64_t seed;
  uint32_t round;
  int32_t* kept_pages;  // optional
  int64_t kept_ld;
  int32_t* freed;
  uint32_t* freed_count;
};

__global__ __launch_bounds__(kThreads) void evict_pages_kernel(PagesArgs a) {
  extern __shared__ int32_t s_dyn[];  // keys [P - pp], old row [P], kept [Kp], kept flag [P]
  __shared__ SelectShared<kThreads> sh;
  __shared__ uint32_t s_scan[kThreads / kWave];
  __shared__ uint32_t s_base;
  const int32_t P = a.P, pp = a.pp, Kp = a.Kp, ps = a.ps;
  const int32_t m = P - pp, kk = Kp - pp;
  uint32_t* s_keys = reinterpret_cast<uint32_t*>(s_dyn);
  int32_t* s_old = s_dyn + m;
  int32_t* s_kept = s_old + P;
  int32_t* s_flag = s_kept + Kp;
  const int64_t g = blockIdx.x;
  const int32_t tid = threadIdx.x;
  int32_t* row = a.pt + g * a.pt_ld;

  const uint64_t request = (uint64_t)(g / a.L), layer = (uint64_t)(g % a.L);
  for (int32_t b = pp + tid; b < P; b += kThreads) {
    const int64_t i = (int64_t)b * ps;  // first slot of page b
    const Philox4x64 r =
        philox4x64_10((uint64_t)(i >> 2), 0u, layer, (request << 32) | a.round, a.seed, 0);
    const uint64_t w = (i & 2) ? ((i & 1) ? r.w[3] : r.w[2]) : ((i & 1) ? r.w[1] : r.w[0]);
    s_keys[b - pp] = draw_key(w);  // word i % 4, with constant indices
  }
  for (int32_t b = tid; b < P; b += kThreads) {
    s_old[b] = row[b];
    s_flag[b] = b < pp;
  }
  for (int32_t j = tid; j < pp; j += kThreads) s_kept[j] = j;
  __syncthreads();

  if (kk > 0) {
    auto key_at = [&](int32_t i) -> uint32_t { return s_keys[i]; };
    uint32_t thr = 0u, need_eq = 0xffffffffu;  // kk == m: keep every candidate page
    if (kk < m) radix_select<24>(key_at, m, kk, sh, thr, need_eq);
    emit_kept(key_at, m, thr, need_eq, sh, [&](uint32_t slot, int32_t i) {
      s_kept[pp + slot] = pp + i;
      s_flag[pp + i] = 1;
    });
  }
  __syncthreads();

  for (int32_t j = tid; j < P; j += kThreads) row[j] = j < Kp ? s_old[s_kept[j]] : -1;
  if (a.kept_pages) {
    int32_t* out = a.kept_pages + g * a.kept_ld;
    for (int32_t j = tid; j < Kp; j += kThreads) out[j] = s_kept[j];
  }
  // evicted pages in page order: output position = evicted pages before b
  if (tid == 0 && P > Kp) s_base = atomicAdd(a.freed_count, (uint32_t)(P - Kp));
  __syncthreads();
  uint32_t carry = 0u;
  for (int32_t b0 = 0; b0 < P; b0 += kThreads) {  // the scan ends with a workgroup barrier
    const int32_t b = b0 + tid;
    const uint32_t out = (b < P && !s_flag[b]) ? 1u : 0u;
    uint32_t total;
    const uint32_t incl = block_inclusive_scan<kThreads>(out, s_scan, &total);
    if (out) a.freed[s_base + carry + incl - 1u] = s_old[b];
    carry += total;
  }
}

}  // namespace

size_t evict_pages_lds_bytes(int32_t P, int32_t pp, int32_t Kp) {
  return (size_t)((P - pp) + P + Kp + P) * sizeof(int32_t);
}

hipError_t launch_evict_pages(int32_t* page_table, int64_t pt_ld, int32_t page_size,
                              int64_t num_groups, int32_t L, int32_t n, int32_t K, int32_t prot,
                              uint64_t seed, uint32_t round, int32_t* kept_pages, int64_t kept_ld,
                              int32_t* freed, uint32_t* freed_count, hipStream_t stream) {
  if (num_groups == 0) return hipSuccess;
  if (num_groups > max_workgroups(kThreads)) return hipErrorInvalidConfiguration;
  PagesArgs a;
  a.pt = page_table;
  a.pt_ld = pt_ld;
  a.ps = page_size;
  a.P = n / page_size;
  a.pp = (prot + page_size - 1) / page_size;
  a.Kp = K / page_size;
  a.L = L;
  a.seed = seed;
  a.round = round;
  a.kept_pages = kept_pages;
  a.kept_ld = kept_ld;
  a.freed = freed;
  a.freed_count = freed_count;
  hipLaunchKernelGGL(evict_pages_kernel, dim3((unsigned)num_groups), dim3(kThreads),
                     evict_pages_lds_bytes(a.P, a.pp, a.Kp), stream, a);
  return hipGetLastError();
}

}  // namespace kvevict
