// Pin + model-wide top-B (GateSight problem statement: B = L*H*round(p*(n-prot))
// entries beyond the protected prefix; KVzip-style global top-B over
// (layer, head, token) scores).
//
// The candidates of each list ([prot, n)) are cut into items of kChunk
// positions, item f = list * chunks + chunk in flat order.
//   init      prompt indices and kept_count = prot for every list; zeroes the
//             histograms, the done counter and the collect counter
//   hist x3   radix histograms of the 11/11/10-bit digits of rank_key(score),
//             restricted to the keys matching the digits chosen so far.  Each
//             workgroup of level l derives the digit of level l - 1 itself
//             from that level's finished histogram and the bucket recorded by
//             the previous kernel (the same computation in every workgroup,
//             so no workgroup has to wait for another), and workgroup 0
//             records the narrowed bucket; a workgroup returns at once if an
//             earlier level took its bucket whole.
//   count     derives the last digit, hence the threshold key T, and writes
//             per-item counts of keys > T and == T; with many items the last
//             count workgroup scans them once into per-item offsets
//   emit      reads T; the item's offset (ties at T go to the lowest list*n + i): the
//             sums over the items before it, or the scanned offset; the
//             per-list kept counts; a ballot/mbcnt chronological emit.
// With at most kCollectItems items the third histogram gets no kernel of its
// own: after two levels the count kernel resolves the second digit, counts per
// item the keys above the 22-bit bucket and in it, adds the bucket's keys to
// the last level's histogram and lists them (item, low 10 bits) while the
// list has room; the emit resolves the last digit and takes the per-item
// counts at T from the list, or, when too many keys share the bucket to list
// them, recounts the items before its own that hold some.
// All counts are integer atomics or scans, so the result is deterministic (the
// collect list's order varies from run to run; only counts over it are used).
//
// Words passed between workgroups of one kernel (the per-item counts and the
// done counter read by the last count workgroup) are written and read only
// with device-scope atomics, which take effect at the device's coherence point
// and need no cache flush (a device-scope fence would write back and
// invalidate every XCD's L2).  Words read only by later kernels of the call
// (histograms, per-item counts, offsets) are read with plain loads: the kernel
// boundary makes them visible.
#include <mutex>

#include "kvevict.h"
#include "kvevict_device.hpp"
#include "kvevict_launch.hpp"

namespace kvevict {
namespace {

constexpr int kThreads = 1024;
static_assert(kThreads == kGlobalThreads, "the grid checks of the fused call");
constexpr int kBinsPerThread = 2048 / kThreads;
static_assert(kBinsPerThread >= 1 && 2048 % kThreads == 0 && 1024 % kThreads == 0,
              "resolve: whole bins per thread");
constexpr int kWaves = kThreads / kWave;
// 8 keys per thread.  Same-process A/B on 64 lists of 32,512 candidates, back to
// back / inside the round: 45.7 / 51.6 us, against 48.9 / 56.5 us with 512
// threads and 16 keys per thread, 55.8 / 61.4 us with 4096-key items on 1024
// threads and 49.3 / 57.6 us with 12,288-key items.
constexpr int32_t kChunk = 8192;

// workspace layout (uint32 words)
static_assert(kGlobalFirstLevelBins == 2048, "first level: key bits [21, 32)");
constexpr int64_t kHist0 = 0;       // 2048 bins, key bits [21, 32)
constexpr int64_t kHist1 = 2048;    // 2048 bins, key bits [10, 21)
constexpr int64_t kHist2 = 4096;    // 1024 bins, key bits [0, 10)
constexpr int64_t kDone = 5184;     // finished workgroups of the count kernel
constexpr int64_t kState = 5188;    // the bucket after levels [0, k): 4 words at kState + 4 (k - 1)
constexpr int64_t kCollected = 5200;  // keys of the 22-bit bucket the count kernel met
constexpr int64_t kArrays = 5248;   // gt[M], eq[M], eqx[M], S[M+1], then the collect list
static_assert(kState + 12 <= kCollected && kCollected < kArrays, "workspace words overlap");
// The collect list: (item << 10) | low 10 key bits of each key in the bucket.
constexpr uint32_t kCollectCap = 4096;
// Items up to which the two-level flow runs.  Its fallback (too many keys in
// the bucket to list) recounts up to all earlier items in every emit
// workgroup, so its cost grows with the square of the items.
constexpr int64_t kCollectItems = 256;
static_assert(kCollectItems << 10 < (1LL << 32), "collect entries fit 32 bits");

enum Mode : int32_t { kNormal = 0, kNone = 1, kAll = 2 };

struct Level {
  int64_t off;
  uint32_t bins;
  int shift;
};
__device__ __forceinline__ Level level_of(int lvl) {
  if (lvl == 0) return {kHist0, 2048u, 21};
  if (lvl == 1) return {kHist1, 2048u, 10};
  return {kHist2, 1024u, 0};
}

__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_dev(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// True in every thread of the workgroup that finishes last among the grid's
// workgroups (counter `done`).  Each wave first waits until all its memory
// operations are acknowledged (s_waitcnt on every counter), so that the
// device-scope atomics of every workgroup that has counted itself are
// performed before the last one reads their words.  (A workgroup-scope fence
// is not enough: it need not wait for global writes at all.)
__device__ bool last_workgroup(uint32_t* done, uint32_t* s_flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) *s_flag = add_dev(done, 1u) == gridDim.x - 1u;
  __syncthreads();
  return *s_flag != 0u;
}

struct GlobalArgs {
  const float* scores;
  int64_t ld;
  int32_t n, prot, chunks;
  int64_t num_lists;
  uint32_t budget;
  int32_t mode;
  uint32_t* ws;
  int32_t* kept_idx;
  int64_t kept_ld;
  int32_t* kept_count;
};

__device__ __forceinline__ void item_range(const GlobalArgs& a, int64_t f, int64_t* list,
                                           int32_t* i0, int32_t* i1) {
  *list = f / a.chunks;
  const int32_t chunk = (int32_t)(f - *list * a.chunks);
  *i0 = a.prot + chunk * kChunk;
  *i1 = min(a.n, *i0 + kChunk);
}

constexpr int kKeysPerThread = kChunk / kThreads;
// Up to this many items, every emit workgroup sums the per-item counts before
// its own item itself; beyond it, the last count workgroup scans them once.
constexpr int64_t kDirectPrefixItems = 8192;

// Loads the item's keys into registers, all loads in flight at once: key u of
// the thread is position i0 + threadIdx.x + u * kThreads (valid if < i1).
__device__ __forceinline__ void load_keys(const float* row, int32_t i0, int32_t i1,
                                          uint32_t* keys) {
#pragma unroll
  for (int u = 0; u < kKeysPerThread; ++u) {
    const int32_t i = i0 + threadIdx.x + u * kThreads;
    keys[u] = (i < i1) ? rank_key(row[i]) : 0u;
  }
}

// The bins of level lvl held by this thread, top bins first: thread t holds
// bins [top - per, top), top = bins - per * t.
__device__ __forceinline__ void load_level_bins(const uint32_t* ws, int lvl, uint32_t* h) {
  const Level L = level_of(lvl);
  const uint32_t per = L.bins / kThreads;
  const uint32_t top = L.bins - per * threadIdx.x;
#pragma unroll
  for (uint32_t b = 0; b < (uint32_t)kBinsPerThread; ++b)
    h[b] = (b < per) ? ws[L.off + top - 1u - b] : 0u;
}

// The digits chosen by levels [0, k): prefix and mask of the bucket that holds
// the budget-th best key, how many keys of that bucket are still to be kept,
// and whether the bucket is kept whole (later levels are then skipped).
struct Thr {
  uint32_t prefix, mask, remaining, whole;
};

// The bucket after levels [0, k), k >= 1, is resolved once per kernel: every
// workgroup of the kernel that reads the finished histogram of level k - 1
// derives it (the same computation in each, so none waits for another) and
// workgroup 0 records it for the later kernels of the call, which read it with
// plain loads after the kernel boundary.
__device__ __forceinline__ Thr load_resolved(const GlobalArgs& a, int k) {
  if (k == 0) return Thr{0u, 0u, a.budget, 0u};
  const uint32_t* s = a.ws + kState + 4 * (k - 1);
  return Thr{s[0], s[1], s[2], s[3]};
}
__device__ __forceinline__ void store_resolved(const GlobalArgs& a, int k, const Thr& t) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    uint32_t* s = a.ws + kState + 4 * (k - 1);
    s[0] = t.prefix;
    s[1] = t.mask;
    s[2] = t.remaining;
    s[3] = t.whole;
  }
}

// Narrows the bucket t of levels [0, lvl) by the digit of level lvl, whose
// bins this thread holds in h.  t is the same in every thread, so a bucket
// already kept whole skips the level in all of them.
__device__ Thr resolve_level(const uint32_t* h, int lvl, Thr t, uint32_t* s_scan, uint32_t* st) {
  if (t.whole) return t;
  const int tid = threadIdx.x;
  const Level L = level_of(lvl);
  const uint32_t per = L.bins / kThreads;
  const uint32_t top = L.bins - per * (uint32_t)tid;
  uint32_t c = 0u;
#pragma unroll
  for (uint32_t b = 0; b < (uint32_t)kBinsPerThread; ++b) c += h[b];
  if (tid == 0) {  // kept if no bin crosses (cannot happen: the bucket holds >= remaining)
    st[0] = t.prefix;
    st[1] = t.mask;
    st[2] = t.remaining;
    st[3] = t.whole;
  }
  uint32_t total;
  const uint32_t incl = block_inclusive_scan<kThreads>(c, s_scan, &total);
  const uint32_t excl = incl - c;
  if (excl < t.remaining && incl >= t.remaining) {
    uint32_t acc = excl;
#pragma unroll
    for (uint32_t b = 0; b < (uint32_t)kBinsPerThread; ++b) {
      if (b < per && acc < t.remaining && acc + h[b] >= t.remaining) {
        const uint32_t left = t.remaining - acc;
        st[0] = t.prefix | ((top - 1u - b) << L.shift);
        st[1] = t.mask | ((L.bins - 1u) << L.shift);
        st[2] = left;
        st[3] = (left == h[b]) ? 1u : 0u;  // the bucket is kept whole
      }
      acc += h[b];
    }
  }
  __syncthreads();  // thread 0's write came before the scan's barriers, the crossing one's after
  return Thr{st[0], st[1], st[2], st[3]};
}

// Threshold key T and how many keys equal to T are kept.
__device__ __forceinline__ void threshold_of(const GlobalArgs& a, const Thr& t, uint32_t* thr,
                                             uint32_t* need_eq) {
  if (a.mode == kAll) {
    *thr = 0u;
    *need_eq = 0xffffffffu;
  } else {
    *thr = t.prefix;
    *need_eq = t.whole ? 0xffffffffu : t.remaining;
  }
}

__global__ __launch_bounds__(kThreads) void global_init_kernel(GlobalArgs a) {
  const int64_t list = blockIdx.x;
  int32_t* out = a.kept_idx + list * a.kept_ld;
  for (int32_t j = threadIdx.x; j < a.prot; j += kThreads) out[j] = j;
  if (threadIdx.x == 0) a.kept_count[list] = a.prot;
  for (int64_t b = list * kThreads + threadIdx.x; b < kArrays; b += gridDim.x * kThreads)
    st_dev(a.ws + b, 0u);
}

__global__ __launch_bounds__(kThreads) void global_hist_kernel(GlobalArgs a, int lvl) {
  __shared__ uint32_t s_hist[2048];
  __shared__ uint32_t s_scan[kWaves];
  __shared__ uint32_t s_state[4];
  int64_t list;
  int32_t i0, i1;
  item_range(a, blockIdx.x, &list, &i0, &i1);
  Thr t = load_resolved(a, lvl > 0 ? lvl - 1 : 0);
  uint32_t h[kBinsPerThread];
  if (lvl > 0) load_level_bins(a.ws, lvl - 1, h);
  uint32_t keys[kKeysPerThread];
  load_keys(a.scores + list * a.ld, i0, i1, keys);  // in flight while the digit resolves
  if (lvl > 0) {
    t = resolve_level(h, lvl - 1, t, s_scan, s_state);
    store_resolved(a, lvl, t);
  }
  if (t.whole) return;  // an earlier level took its bucket whole
  const Level L = level_of(lvl);
  for (uint32_t b = threadIdx.x; b < L.bins; b += kThreads) s_hist[b] = 0u;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kKeysPerThread; ++u) {
    const uint32_t k = keys[u];
    if (i0 + (int32_t)threadIdx.x + u * kThreads < i1 && (k & t.mask) == t.prefix)
      atomicAdd(&s_hist[(k >> L.shift) & (L.bins - 1u)], 1u);
  }
  __syncthreads();
  for (uint32_t b = threadIdx.x; b < L.bins; b += kThreads) {
    const uint32_t h = s_hist[b];
    if (h) add_dev(a.ws + L.off + b, h);
  }
}

// Emits the kept indices of an item whose keys are in registers: keys > thr,
// and keys == thr while fewer than need_eq of them come before in flat order
// (eq0 of them lie in earlier items).  `out` points at the item's first slot.
// Key u of a thread sits at item position u*kThreads + threadIdx.x, so the
// chronological order runs over (u, wave, lane): every wave ballots all its
// keys first, one wave scans the per-(u, wave) counts, and each key's slot is
// its scanned prefix plus the set lanes below it (two barriers in all).
__device__ __forceinline__ void emit_item(const uint32_t* keys, int32_t i0, int32_t i1,
                                          uint32_t thr, uint32_t need_eq, uint32_t eq0,
                                          int32_t* out, uint32_t* s_cnt) {
  constexpr int kSlots = kKeysPerThread * kWaves;  // (u, wave) slots per kind
  static_assert(2 * kSlots == 4 * kWave, "the scan gives four counts to each lane of a wave");
  const uint32_t taken0 = min(eq0, need_eq);
  const int wave = threadIdx.x / kWave;
  const uint32_t lane = lane_id();
  uint64_t bg[kKeysPerThread], be[kKeysPerThread];
#pragma unroll
  for (int u = 0; u < kKeysPerThread; ++u) {
    const bool valid = i0 + (int32_t)threadIdx.x + u * kThreads < i1;
    bg[u] = __ballot(valid && keys[u] > thr);
    be[u] = __ballot(valid && keys[u] == thr);
    if (lane == 0) {
      s_cnt[u * kWaves + wave] = (uint32_t)__popcll(bg[u]);
      s_cnt[kSlots + u * kWaves + wave] = (uint32_t)__popcll(be[u]);
    }
  }
  __syncthreads();
  if (wave == 0) {  // exclusive prefixes, gt counts and eq counts separately
    uint32_t c[4], run = 0u;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c[q] = s_cnt[lane * 4 + q];
      run += c[q];
    }
    // lanes [0, 32) hold the gt counts, [32, 64) the eq counts
    uint32_t incl = run;
#pragma unroll
    for (int d = 1; d < kWave / 2; d <<= 1) {
      const uint32_t t = __shfl_up(incl, d, kWave / 2);
      if ((lane & (kWave / 2 - 1)) >= (uint32_t)d) incl += t;
    }
    uint32_t pre = incl - run;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s_cnt[2 * kSlots + lane * 4 + q] = pre;
      pre += c[q];
    }
  }
  __syncthreads();
  const uint32_t* pre_gt = s_cnt + 2 * kSlots;
  const uint32_t* pre_eq = pre_gt + kSlots;
#pragma unroll
  for (int u = 0; u < kKeysPerThread; ++u) {
    const bool gt = (bg[u] >> lane) & 1u;
    const bool eq = (be[u] >> lane) & 1u;
    const uint32_t gt_before = pre_gt[u * kWaves + wave] + count_below(bg[u]);
    const uint32_t eq_before = eq0 + pre_eq[u * kWaves + wave] + count_below(be[u]);  // flat order
    if (gt || (eq && eq_before < need_eq))
      out[gt_before + min(eq_before, need_eq) - taken0] = i0 + (int32_t)threadIdx.x + u * kThreads;
  }
}

__device__ __forceinline__ void count_item(const uint32_t* keys, int32_t i0, int32_t i1,
                                           uint32_t thr, uint32_t* gt, uint32_t* eq) {
  uint32_t g = 0u, e = 0u;
#pragma unroll
  for (int u = 0; u < kKeysPerThread; ++u) {
    const bool valid = i0 + (int32_t)threadIdx.x + u * kThreads < i1;
    g += (valid && keys[u] > thr) ? 1u : 0u;
    e += (valid && keys[u] == thr) ? 1u : 0u;
  }
  *gt = g;
  *eq = e;
}

// Per-item counts of keys > T and == T.  With more than kDirectPrefixItems
// items, the last workgroup then scans them in flat order into per-item
// offsets and writes the per-list counts.
__global__ __launch_bounds__(kThreads) void global_count_kernel(GlobalArgs a, int levels) {
  __shared__ uint32_t s_scan[kWaves];
  __shared__ uint32_t s_state[4];
  __shared__ uint32_t s_flag;
  const int64_t f = blockIdx.x;
  const int64_t M = a.num_lists * a.chunks;
  uint32_t* gt_arr = a.ws + kArrays;
  uint32_t* eq_arr = gt_arr + M;
  uint32_t* eqx = gt_arr + 2 * M;
  uint32_t* S = gt_arr + 3 * M;
  int64_t list;
  int32_t i0, i1;
  item_range(a, f, &list, &i0, &i1);
  Thr t = load_resolved(a, levels > 0 ? levels - 1 : 0);
  uint32_t h[kBinsPerThread];
  if (levels > 0) load_level_bins(a.ws, levels - 1, h);
  uint32_t keys[kKeysPerThread];
  load_keys(a.scores + list * a.ld, i0, i1, keys);
  if (levels > 0) {
    t = resolve_level(h, levels - 1, t, s_scan, s_state);
    store_resolved(a, levels, t);
  }
  uint32_t thr, need_eq;
  threshold_of(a, t, &thr, &need_eq);
  uint32_t gt, eq;
  count_item(keys, i0, i1, thr, &gt, &eq);
  gt = block_sum<kThreads>(gt, s_scan);
  eq = block_sum<kThreads>(eq, s_scan);
  if (threadIdx.x == 0) {
    st_dev(gt_arr + f, gt);
    st_dev(eq_arr + f, eq);
  }
  if (M <= kDirectPrefixItems || !last_workgroup(a.ws + kDone, &s_flag)) return;

  // the last workgroup: scans in flat order and per-list counts
  const int tid = threadIdx.x;
  uint32_t carry = 0u;
  for (int64_t base = 0; base < M; base += kThreads) {
    const int64_t g = base + tid;
    const uint32_t e = (g < M) ? ld_dev(eq_arr + g) : 0u;
    uint32_t total;
    const uint32_t incl = block_inclusive_scan<kThreads>(e, s_scan, &total);
    if (g < M) st_dev(eqx + g, carry + incl - e);
    carry += total;
  }
  __syncthreads();
  carry = 0u;
  for (int64_t base = 0; base < M; base += kThreads) {
    const int64_t g = base + tid;
    uint32_t k = 0u;
    if (g < M) {
      const uint32_t x = ld_dev(eqx + g);
      const uint32_t room = (need_eq > x) ? need_eq - x : 0u;
      k = ld_dev(gt_arr + g) + min(ld_dev(eq_arr + g), room);
    }
    uint32_t total;
    const uint32_t incl = block_inclusive_scan<kThreads>(k, s_scan, &total);
    if (g < M) st_dev(S + g, carry + incl - k);
    carry += total;
  }
  if (tid == 0) st_dev(S + M, carry);
  __syncthreads();
  for (int64_t l = tid; l < a.num_lists; l += kThreads)
    a.kept_count[l] = a.prot + (int32_t)(ld_dev(S + (l + 1) * a.chunks) - ld_dev(S + l * a.chunks));
}

__global__ __launch_bounds__(kThreads) void global_emit_kernel(GlobalArgs a, int levels) {
  __shared__ uint32_t s_scan[kWaves];
  __shared__ uint32_t s_cnt[4 * kKeysPerThread * kWaves];
  const int64_t f = blockIdx.x;
  const int64_t M = a.num_lists * a.chunks;
  const bool direct = M <= kDirectPrefixItems;
  int64_t list;
  int32_t i0, i1;
  item_range(a, f, &list, &i0, &i1);
  // everything this workgroup reads is issued up front: the resolved bucket,
  // the item's keys and the per-item counts or offsets written by earlier
  // kernels (plain loads: the kernel boundary makes them visible)
  const Thr t = load_resolved(a, levels);
  uint32_t keys[kKeysPerThread];
  load_keys(a.scores + list * a.ld, i0, i1, keys);
  const uint32_t* gt_arr = a.ws + kArrays;
  const uint32_t* eq_arr = gt_arr + M;
  const int64_t ls = list * a.chunks;
  uint32_t e_all = 0u, gt_in = 0u, e_in = 0u, eq0, offset;
  if (direct) {  // sums over the items before f: all of them for eq, f's list for gt and eq
    for (int64_t g = threadIdx.x; g < f; g += kThreads) {
      const uint32_t e = eq_arr[g];
      e_all += e;
      if (g >= ls) {
        gt_in += gt_arr[g];
        e_in += e;
      }
    }
  } else {
    eq0 = gt_arr[2 * M + f];                     // eqx[f]
    offset = gt_arr[3 * M + f] - gt_arr[3 * M + ls];  // S[f] - S[ls]
  }
  uint32_t thr, need_eq;
  threshold_of(a, t, &thr, &need_eq);
  if (direct) {
    eq0 = block_sum<kThreads>(e_all, s_scan);
    gt_in = block_sum<kThreads>(gt_in, s_scan);
    e_in = block_sum<kThreads>(e_in, s_scan);
    // keys == T are kept in flat order, so the run [ls, f) keeps the first
    // (need_eq - eq before ls) of its e_in, clamped to [0, e_in]
    const uint32_t eq_ls = eq0 - e_in;
    const uint32_t room_ls = (need_eq > eq_ls) ? need_eq - eq_ls : 0u;
    offset = gt_in + min(e_in, room_ls);
    if (f - ls == a.chunks - 1 && threadIdx.x == 0) {  // last item of its list
      const uint32_t room_f = (need_eq > eq0) ? need_eq - eq0 : 0u;
      a.kept_count[list] = a.prot + (int32_t)(offset + gt_arr[f] + min(eq_arr[f], room_f));
    }
  }
  emit_item(keys, i0, i1, thr, need_eq, eq0, a.kept_idx + list * a.kept_ld + a.prot + offset,
            s_cnt);
}

// Two-level flow, count: resolves the second digit (the bucket of the top 22
// key bits).  A bucket kept whole fixes T exactly, and the item's counts of
// keys > T and == T are stored as in the three-level flow.  Otherwise gt[f]
// is the count of keys above the bucket and eq[f] of keys in it; the bucket's
// keys add to the third level's bins and are listed while the list has room
// (the counter keeps counting past it).
__global__ __launch_bounds__(kThreads) void global_count_collect_kernel(GlobalArgs a) {
  __shared__ uint32_t s_hist[1024];
  __shared__ uint32_t s_scan[kWaves];
  __shared__ uint32_t s_state[4];
  __shared__ uint32_t s_base;
  const int tid = threadIdx.x;
  const int64_t f = blockIdx.x;
  const int64_t M = a.num_lists * a.chunks;
  uint32_t* gt_arr = a.ws + kArrays;
  uint32_t* eq_arr = gt_arr + M;
  int64_t list;
  int32_t i0, i1;
  item_range(a, f, &list, &i0, &i1);
  Thr t = load_resolved(a, 1);
  uint32_t h[kBinsPerThread];
  load_level_bins(a.ws, 1, h);
  uint32_t keys[kKeysPerThread];
  load_keys(a.scores + list * a.ld, i0, i1, keys);
  t = resolve_level(h, 1, t, s_scan, s_state);
  store_resolved(a, 2, t);
  uint32_t gt = 0u, eq = 0u;
  if (t.whole) {
    uint32_t thr, need_eq;
    threshold_of(a, t, &thr, &need_eq);
    count_item(keys, i0, i1, thr, &gt, &eq);
    gt = block_sum<kThreads>(gt, s_scan);
    eq = block_sum<kThreads>(eq, s_scan);
    if (tid == 0) {
      st_dev(gt_arr + f, gt);
      st_dev(eq_arr + f, eq);
    }
    return;
  }
  for (int b = tid; b < 1024; b += kThreads) s_hist[b] = 0u;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kKeysPerThread; ++u) {
    if (i0 + tid + u * kThreads >= i1) continue;
    const uint32_t top = keys[u] & t.mask;
    if (top > t.prefix) {
      ++gt;
    } else if (top == t.prefix) {
      ++eq;
      atomicAdd(&s_hist[keys[u] & 1023u], 1u);
    }
  }
  __syncthreads();
  for (int b = tid; b < 1024; b += kThreads) {
    const uint32_t c = s_hist[b];
    if (c) add_dev(a.ws + kHist2 + b, c);
  }
  uint32_t total_eq;
  const uint32_t eq_before = block_inclusive_scan<kThreads>(eq, s_scan, &total_eq) - eq;
  gt = block_sum<kThreads>(gt, s_scan);
  if (tid == 0) {
    st_dev(gt_arr + f, gt);
    st_dev(eq_arr + f, total_eq);
    s_base = total_eq ? add_dev(a.ws + kCollected, total_eq) : 0u;
  }
  __syncthreads();
  uint32_t slot = s_base + eq_before;
  uint32_t* lst = a.ws + kArrays + 4 * M + 1;
#pragma unroll
  for (int u = 0; u < kKeysPerThread; ++u) {
    if (i0 + tid + u * kThreads >= i1 || (keys[u] & t.mask) != t.prefix) continue;
    if (slot < kCollectCap) lst[slot] = ((uint32_t)f << 10) | (keys[u] & 1023u);
    ++slot;
  }
}

// Two-level flow, emit: resolves the last digit from the third level's bins
// (unless the bucket was kept whole), then the item's offset as in the direct
// three-level emit, with the per-item counts at T taken from the list (or by
// recounting the earlier items that hold bucket keys when it overflowed).
__global__ __launch_bounds__(kThreads) void global_emit_collect_kernel(GlobalArgs a) {
  __shared__ uint32_t s_scan[kWaves];
  __shared__ uint32_t s_cnt[4 * kKeysPerThread * kWaves];
  __shared__ uint32_t s_state[4];
  const int tid = threadIdx.x;
  const int64_t f = blockIdx.x;
  const int64_t M = a.num_lists * a.chunks;
  int64_t list;
  int32_t i0, i1;
  item_range(a, f, &list, &i0, &i1);
  Thr t = load_resolved(a, 2);
  uint32_t h[kBinsPerThread];
  load_level_bins(a.ws, 2, h);
  uint32_t keys[kKeysPerThread];
  load_keys(a.scores + list * a.ld, i0, i1, keys);
  const uint32_t* gt_arr = a.ws + kArrays;
  const uint32_t* eq_arr = gt_arr + M;
  const uint32_t collected = a.ws[kCollected];
  const bool whole = t.whole != 0u;
  const int64_t ls = list * a.chunks;
  // over the items before f: gt of [ls, f) (exact if whole, else above the
  // bucket), and, if whole, eq of all of them and of [ls, f)
  uint32_t g_in = 0u, e_all = 0u, e_in = 0u;
  for (int64_t g = tid; g < f; g += kThreads) {
    const uint32_t e = whole ? eq_arr[g] : 0u;
    e_all += e;
    if (g >= ls) {
      g_in += gt_arr[g];
      e_in += e;
    }
  }
  t = resolve_level(h, 2, t, s_scan, s_state);  // unchanged when whole
  uint32_t thr, need_eq;
  threshold_of(a, t, &thr, &need_eq);
  if (!whole) {
    const uint32_t d = thr & 1023u;
    if (collected <= kCollectCap) {
      const uint32_t* lst = a.ws + kArrays + 4 * M + 1;
      for (uint32_t e = tid; e < collected; e += kThreads) {
        const uint32_t x = lst[e];
        const int64_t g = x >> 10;
        const uint32_t low = x & 1023u;
        if (g >= f) continue;
        if (low == d) {
          ++e_all;
          if (g >= ls) ++e_in;
        } else if (low > d && g >= ls) {
          ++g_in;
        }
      }
    } else {
      for (int64_t g = 0; g < f; ++g) {
        if (eq_arr[g] == 0u) continue;  // no key of item g is in the bucket
        int64_t gl;
        int32_t j0, j1;
        item_range(a, g, &gl, &j0, &j1);
        uint32_t k2[kKeysPerThread];
        load_keys(a.scores + gl * a.ld, j0, j1, k2);
        uint32_t cg, ce;
        count_item(k2, j0, j1, thr, &cg, &ce);
        e_all += ce;
        if (g >= ls) {
          e_in += ce;
          g_in += cg;  // the exact count replaces the keys above the bucket, added once
          if (tid == 0) g_in -= gt_arr[g];
        }
      }
    }
  }
  const uint32_t eq0 = block_sum<kThreads>(e_all, s_scan);
  g_in = block_sum<kThreads>(g_in, s_scan);
  e_in = block_sum<kThreads>(e_in, s_scan);
  // keys == T are kept in flat order, so the run [ls, f) keeps the first
  // (need_eq - eq before ls) of its e_in, clamped to [0, e_in]
  const uint32_t eq_ls = eq0 - e_in;
  const uint32_t room_ls = (need_eq > eq_ls) ? need_eq - eq_ls : 0u;
  const uint32_t offset = g_in + min(e_in, room_ls);
  if (f - ls == a.chunks - 1) {  // last item of its list: the list's kept count
    uint32_t cg, ce;
    count_item(keys, i0, i1, thr, &cg, &ce);
    cg = block_sum<kThreads>(cg, s_scan);
    ce = block_sum<kThreads>(ce, s_scan);
    if (tid == 0) {
      const uint32_t room_f = (need_eq > eq0) ? need_eq - eq0 : 0u;
      a.kept_count[list] = a.prot + (int32_t)(offset + cg + min(ce, room_f));
    }
  }
  emit_item(keys, i0, i1, thr, need_eq, eq0, a.kept_idx + list * a.kept_ld + a.prot + offset,
            s_cnt);
}

}  // namespace

size_t select_global_workspace_bytes(int64_t num_lists, int32_t n, int32_t prot) {
  const int64_t m = n - prot;
  const int64_t chunks = (m + kChunk - 1) / kChunk;
  const int64_t M = num_lists * chunks;
  const int64_t words = kArrays + 4 * M + 1 + kCollectCap;
  return (size_t)((words * 4 + 255) / 256 * 256);
}

// --- the workspace of the allocation-free entry point ------------------------------
// One static device array per GPU, sized for kScratchItems items of kChunk
// candidates (the workspace select_global_workspace_bytes asks for at that many
// items).  Every call on a GPU uses that GPU's copy; the select clears what it
// needs at the start of each call (init kernel), so nothing carries over.
constexpr int64_t kScratchItems = 65536;
constexpr size_t kScratchBytes =
    (size_t)(((kArrays + 4 * kScratchItems + 1 + kCollectCap) * 4 + 255) / 256 * 256);
static_assert(kScratchBytes == KVEVICT_SELECT_GLOBAL_NOALLOC_BYTES,
              "the header states the scratch size");

namespace {
static __device__ __align__(256) uint32_t scratch[kScratchBytes / 4];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch`, per device
}  // namespace

hipError_t select_global_scratch(void** ptr, size_t* bytes) {
  *ptr = nullptr;
  *bytes = kScratchBytes;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {  // first call on this device, which is current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

namespace {

GlobalArgs global_args(int32_t* kept_idx, int64_t kept_ld, int32_t* kept_count,
                       const float* scores, int64_t ld, int64_t num_lists, int32_t n,
                       int32_t prot, int64_t budget, void* workspace) {
  const int64_t m = n - prot;
  GlobalArgs a;
  a.scores = scores;
  a.ld = ld;
  a.n = n;
  a.prot = prot;
  a.chunks = (int32_t)((m + kChunk - 1) / kChunk);
  a.num_lists = num_lists;
  a.budget = (uint32_t)budget;
  a.mode = (budget <= 0) ? kNone : (budget >= num_lists * m ? kAll : kNormal);
  a.ws = static_cast<uint32_t*>(workspace);
  a.kept_idx = kept_idx;
  a.kept_ld = kept_ld;
  a.kept_count = kept_count;
  return a;
}

}  // namespace

uint32_t* select_global_first_level_bins(int64_t num_lists, int32_t n, int32_t prot,
                                         int64_t budget, void* workspace) {
  const int64_t m = n - prot;
  const bool levels = num_lists > 0 && m > 0 && budget > 0 && budget < num_lists * m;
  return levels ? static_cast<uint32_t*>(workspace) + kHist0 : nullptr;
}

hipError_t launch_select_global_init(int32_t* kept_idx, int64_t kept_ld, int32_t* kept_count,
                                     int64_t num_lists, int32_t n, int32_t prot, int64_t budget,
                                     void* workspace, hipStream_t stream) {
  if (num_lists == 0) return hipSuccess;
  if (num_lists > max_workgroups(kThreads)) return hipErrorInvalidConfiguration;
  const GlobalArgs a = global_args(kept_idx, kept_ld, kept_count, nullptr, n, num_lists, n, prot,
                                   budget, workspace);
  hipLaunchKernelGGL(global_init_kernel, dim3((unsigned)num_lists), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_select_global(int32_t* kept_idx, int64_t kept_ld, int32_t* kept_count,
                                const float* scores, int64_t ld, int64_t num_lists, int32_t n,
                                int32_t prot, int64_t budget, void* workspace,
                                hipStream_t stream, bool first_level_done) {
  if (num_lists == 0) return hipSuccess;
  if (num_lists > max_workgroups(kThreads)) return hipErrorInvalidConfiguration;
  const GlobalArgs a = global_args(kept_idx, kept_ld, kept_count, scores, ld, num_lists, n, prot,
                                   budget, workspace);
  hipError_t e;
  if (!first_level_done) {
    hipLaunchKernelGGL(global_init_kernel, dim3((unsigned)num_lists), dim3(kThreads), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const unsigned items = (unsigned)(num_lists * a.chunks);
  if (items == 0 || a.mode == kNone) return hipSuccess;  // the prompts are the whole result
  if (a.mode == kNormal && (int64_t)items <= kCollectItems) {  // two histogram levels
    for (int lvl = (first_level_done ? 1 : 0); lvl < 2; ++lvl) {
      hipLaunchKernelGGL(global_hist_kernel, dim3(items), dim3(kThreads), 0, stream, a, lvl);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(global_count_collect_kernel, dim3(items), dim3(kThreads), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(global_emit_collect_kernel, dim3(items), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
  }
  const int levels = (a.mode == kNormal) ? 3 : 0;
  for (int lvl = (first_level_done ? 1 : 0); lvl < levels; ++lvl) {
    hipLaunchKernelGGL(global_hist_kernel, dim3(items), dim3(kThreads), 0, stream, a, lvl);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(global_count_kernel, dim3(items), dim3(kThreads), 0, stream, a, levels);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(global_emit_kernel, dim3(items), dim3(kThreads), 0, stream, a, levels);
  return hipGetLastError();
}

}  // namespace kvevict
