// Pin + model-wide top-B (GateSight problem statement: B = L*H*round(p*(n-prot))
// entries beyond the protected prefix; KVzip-style global top-B over
// (layer, head, token) scores).
//
// The candidates of each list ([prot, n)) are cut into chunks of kChunk
// positions; one workgroup owns one (list, chunk) in every kernel below.
//   init      prompt indices of every list; zero the histograms
//   hist x3   radix histograms of the 11/11/10-bit digits of rank_key(score),
//             restricted to the keys matching the digits chosen so far;
//             each workgroup resolves the earlier digits itself from the
//             finished histograms (a 2048-bin scan), so no extra launches
//   count     threshold key T and the number of keys equal to T to keep;
//             per-chunk counts of keys > T and == T
//   scan      one workgroup: exclusive scans over the chunks in flat order
//             (ties at T go to the lowest list*n + i), per-list kept counts
//   emit      ballot/mbcnt chronological emit of every chunk at its offset
// All counts are integer atomics or scans, so the result is deterministic.
#include "kvevict_device.hpp"
#include "kvevict_launch.hpp"

namespace kvevict {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int32_t kChunk = 4096;

// workspace layout (uint32 words)
constexpr int64_t kHist0 = 0;      // 2048 bins, key bits [21, 32)
constexpr int64_t kHist1 = 2048;   // 2048 bins, key bits [10, 21)
constexpr int64_t kHist2 = 4096;   // 1024 bins, key bits [0, 10)
constexpr int64_t kState = 5120;   // {T, need_eq}
constexpr int64_t kArrays = 5128;  // gt[M], eq[M], eqx[M], S[M+1]

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

struct Resolved {
  uint32_t prefix, mask, remaining;
  bool whole_bucket;
};

// Walks the finished histograms of levels [0, levels) from the top bin down
// and returns the chosen digits.  Called by all threads of a workgroup.
__device__ Resolved resolve(const uint32_t* ws, int levels, uint32_t budget, uint32_t* s_scan,
                            uint32_t* s_pick) {
  Resolved r{0u, 0u, budget, false};
  const int tid = threadIdx.x;
  for (int lvl = 0; lvl < levels; ++lvl) {
    const Level L = level_of(lvl);
    const uint32_t* hist = ws + L.off;
    const uint32_t per = L.bins / kThreads;  // 8 or 4 bins per thread, top first
    const uint32_t top = L.bins - per * (uint32_t)tid;  // exclusive upper bin
    uint32_t c = 0u;
    for (uint32_t b = 0; b < per; ++b) c += hist[top - 1u - b];
    uint32_t total;
    const uint32_t incl = block_inclusive_scan<kThreads>(c, s_scan, &total);
    const uint32_t excl = incl - c;
    if (excl < r.remaining && incl >= r.remaining) {
      uint32_t acc = excl;
      for (uint32_t b = 0; b < per; ++b) {
        const uint32_t bin = top - 1u - b;
        const uint32_t h = hist[bin];
        if (acc + h >= r.remaining) {
          s_pick[0] = bin;
          s_pick[1] = r.remaining - acc;
          s_pick[2] = h;
          break;
        }
        acc += h;
      }
    }
    __syncthreads();
    const uint32_t digit = s_pick[0];
    const uint32_t cnt = s_pick[2];
    r.remaining = s_pick[1];
    r.prefix |= digit << L.shift;
    r.mask |= (L.bins - 1u) << L.shift;
    __syncthreads();
    if (r.remaining == cnt) {
      r.whole_bucket = true;
      break;
    }
  }
  return r;
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

__global__ __launch_bounds__(kThreads) void global_init_kernel(GlobalArgs a) {
  const int64_t list = blockIdx.x;
  int32_t* out = a.kept_idx + list * a.kept_ld;
  for (int32_t j = threadIdx.x; j < a.prot; j += kThreads) out[j] = j;
  if (list == 0)
    for (int32_t b = threadIdx.x; b < (int32_t)kArrays; b += kThreads) a.ws[b] = 0u;
}

__global__ __launch_bounds__(kThreads) void global_hist_kernel(GlobalArgs a, int lvl) {
  __shared__ uint32_t s_hist[2048];
  __shared__ uint32_t s_scan[kWaves];
  __shared__ uint32_t s_pick[3];
  const int64_t list = blockIdx.x / a.chunks;
  const int32_t chunk = blockIdx.x % a.chunks;
  const Resolved r = resolve(a.ws, lvl, a.budget, s_scan, s_pick);
  if (lvl > 0 && r.whole_bucket) return;
  const Level L = level_of(lvl);
  for (uint32_t b = threadIdx.x; b < L.bins; b += kThreads) s_hist[b] = 0u;
  __syncthreads();
  const float* row = a.scores + list * a.ld;
  const int32_t i0 = a.prot + chunk * kChunk;
  const int32_t i1 = min(a.n, i0 + kChunk);
  for (int32_t i = i0 + threadIdx.x; i < i1; i += kThreads) {
    const uint32_t k = rank_key(row[i]);
    if ((k & r.mask) == r.prefix) atomicAdd(&s_hist[(k >> L.shift) & (L.bins - 1u)], 1u);
  }
  __syncthreads();
  for (uint32_t b = threadIdx.x; b < L.bins; b += kThreads) {
    const uint32_t h = s_hist[b];
    if (h) atomicAdd(&a.ws[L.off + b], h);
  }
}

__device__ __forceinline__ void threshold(const GlobalArgs& a, uint32_t* s_scan, uint32_t* s_pick,
                                          uint32_t* thr, uint32_t* need_eq) {
  if (a.mode == kNone) {  // keep no candidate: no key exceeds or equals T with need_eq = 0
    *thr = 0xffffffffu;
    *need_eq = 0u;
  } else if (a.mode == kAll) {
    *thr = 0u;
    *need_eq = 0xffffffffu;
  } else {
    const Resolved r = resolve(a.ws, 3, a.budget, s_scan, s_pick);
    *thr = r.prefix;
    *need_eq = r.whole_bucket ? 0xffffffffu : r.remaining;
  }
}

__global__ __launch_bounds__(kThreads) void global_count_kernel(GlobalArgs a) {
  __shared__ uint32_t s_scan[kWaves];
  __shared__ uint32_t s_pick[3];
  const int64_t list = blockIdx.x / a.chunks;
  const int32_t chunk = blockIdx.x % a.chunks;
  uint32_t thr, need_eq;
  threshold(a, s_scan, s_pick, &thr, &need_eq);
  const float* row = a.scores + list * a.ld;
  const int32_t i0 = a.prot + chunk * kChunk;
  const int32_t i1 = min(a.n, i0 + kChunk);
  uint32_t gt = 0u, eq = 0u;
  for (int32_t i = i0 + threadIdx.x; i < i1; i += kThreads) {
    const uint32_t k = rank_key(row[i]);
    gt += (k > thr) ? 1u : 0u;
    eq += (k == thr) ? 1u : 0u;
  }
  gt = block_sum<kThreads>(gt, s_scan);
  eq = block_sum<kThreads>(eq, s_scan);
  const int64_t M = a.num_lists * a.chunks;
  const int64_t f = (int64_t)blockIdx.x;
  if (threadIdx.x == 0) {
    a.ws[kArrays + f] = gt;
    a.ws[kArrays + M + f] = eq;
    if (blockIdx.x == 0) {
      a.ws[kState + 0] = thr;
      a.ws[kState + 1] = need_eq;
    }
  }
}

__global__ __launch_bounds__(1024) void global_scan_kernel(GlobalArgs a) {
  constexpr int NT = 1024;
  __shared__ uint32_t s_scan[NT / kWave];
  const int64_t M = a.num_lists * a.chunks;
  const uint32_t* gt = a.ws + kArrays;
  const uint32_t* eq = gt + M;
  uint32_t* eqx = a.ws + kArrays + 2 * M;
  uint32_t* S = a.ws + kArrays + 3 * M;
  const uint32_t need_eq = (M > 0) ? a.ws[kState + 1] : 0u;
  uint32_t carry = 0u;
  for (int64_t base = 0; base < M; base += NT) {
    const int64_t f = base + threadIdx.x;
    const uint32_t e = (f < M) ? eq[f] : 0u;
    uint32_t total;
    const uint32_t incl = block_inclusive_scan<NT>(e, s_scan, &total);
    if (f < M) eqx[f] = carry + incl - e;
    carry += total;
  }
  __syncthreads();
  carry = 0u;
  for (int64_t base = 0; base < M; base += NT) {
    const int64_t f = base + threadIdx.x;
    uint32_t k = 0u;
    if (f < M) {
      const uint32_t x = eqx[f];
      const uint32_t room = (need_eq > x) ? need_eq - x : 0u;
      k = gt[f] + min(eq[f], room);
    }
    uint32_t total;
    const uint32_t incl = block_inclusive_scan<NT>(k, s_scan, &total);
    if (f < M) S[f] = carry + incl - k;
    carry += total;
  }
  if (threadIdx.x == 0) S[M] = carry;
  __syncthreads();
  for (int64_t list = threadIdx.x; list < a.num_lists; list += NT) {
    uint32_t kept = 0u;
    if (a.chunks > 0) kept = S[(list + 1) * a.chunks] - S[list * a.chunks];
    a.kept_count[list] = a.prot + (int32_t)kept;
  }
}

__global__ __launch_bounds__(kThreads) void global_emit_kernel(GlobalArgs a) {
  __shared__ uint32_t s_tile[2 * kWaves];
  const int64_t list = blockIdx.x / a.chunks;
  const int32_t chunk = blockIdx.x % a.chunks;
  const int64_t M = a.num_lists * a.chunks;
  const int64_t f = (int64_t)blockIdx.x;
  const uint32_t thr = a.ws[kState + 0];
  const uint32_t need_eq = a.ws[kState + 1];
  const uint32_t* eqx = a.ws + kArrays + 2 * M;
  const uint32_t* S = a.ws + kArrays + 3 * M;
  const uint32_t eq0 = eqx[f];
  const uint32_t taken0 = min(eq0, need_eq);
  int32_t* out = a.kept_idx + list * a.kept_ld + a.prot + (S[f] - S[list * a.chunks]);
  const float* row = a.scores + list * a.ld;
  const int32_t i0 = a.prot + chunk * kChunk;
  const int32_t i1 = min(a.n, i0 + kChunk);
  const int wave = threadIdx.x / kWave;
  uint32_t carry_gt = 0u, carry_eq = 0u;
  for (int32_t base = i0; base < i1; base += kThreads) {
    const int32_t i = base + threadIdx.x;
    const bool valid = i < i1;
    const uint32_t k = valid ? rank_key(row[i]) : 0u;
    const bool gt = valid && k > thr;
    const bool eq = valid && k == thr;
    const uint64_t bg = __ballot(gt);
    const uint64_t be = __ballot(eq);
    if (lane_id() == 0) {
      s_tile[wave] = (uint32_t)__popcll(bg);
      s_tile[kWaves + wave] = (uint32_t)__popcll(be);
    }
    __syncthreads();
    uint32_t pre_gt = 0u, pre_eq = 0u, tot_gt = 0u, tot_eq = 0u;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t g = s_tile[w], e = s_tile[kWaves + w];
      pre_gt += (w < wave) ? g : 0u;
      pre_eq += (w < wave) ? e : 0u;
      tot_gt += g;
      tot_eq += e;
    }
    __syncthreads();
    const uint32_t gt_before = carry_gt + pre_gt + count_below(bg);
    const uint32_t eq_before = eq0 + carry_eq + pre_eq + count_below(be);  // flat order
    if (gt || (eq && eq_before < need_eq)) out[gt_before + min(eq_before, need_eq) - taken0] = i;
    carry_gt += tot_gt;
    carry_eq += tot_eq;
  }
}

}  // namespace

size_t select_global_workspace_bytes(int64_t num_lists, int32_t n, int32_t prot) {
  const int64_t m = n - prot;
  const int64_t chunks = (m + kChunk - 1) / kChunk;
  const int64_t M = num_lists * chunks;
  const int64_t words = kArrays + 4 * M + 1;
  return (size_t)((words * 4 + 255) / 256 * 256);
}

hipError_t launch_select_global(int32_t* kept_idx, int64_t kept_ld, int32_t* kept_count,
                                const float* scores, int64_t ld, int64_t num_lists, int32_t n,
                                int32_t prot, int64_t budget, void* workspace,
                                hipStream_t stream) {
  if (num_lists == 0) return hipSuccess;
  const int64_t m = n - prot;
  const int32_t chunks = (int32_t)((m + kChunk - 1) / kChunk);
  GlobalArgs a;
  a.scores = scores;
  a.ld = ld;
  a.n = n;
  a.prot = prot;
  a.chunks = chunks;
  a.num_lists = num_lists;
  a.budget = (uint32_t)budget;
  a.mode = (budget <= 0) ? kNone : (budget >= num_lists * m ? kAll : kNormal);
  a.ws = static_cast<uint32_t*>(workspace);
  a.kept_idx = kept_idx;
  a.kept_ld = kept_ld;
  a.kept_count = kept_count;

  hipLaunchKernelGGL(global_init_kernel, dim3((unsigned)num_lists), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned blocks = (unsigned)(num_lists * chunks);
  if (blocks > 0 && a.mode == kNormal) {
    for (int lvl = 0; lvl < 3; ++lvl) {
      hipLaunchKernelGGL(global_hist_kernel, dim3(blocks), dim3(kThreads), 0, stream, a, lvl);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (blocks > 0) {
    hipLaunchKernelGGL(global_count_kernel, dim3(blocks), dim3(kThreads), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(global_scan_kernel, dim3(1), dim3(1024), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (blocks > 0) {
    hipLaunchKernelGGL(global_emit_kernel, dim3(blocks), dim3(kThreads), 0, stream, a);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace kvevict
