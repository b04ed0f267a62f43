// Pin + per-head top-K ("Random Attention" blog summary, Algorithm 1: prompt
// pinned to +inf, top-K per KV head, return the keep set; also fused with the
// random draw itself), with the per-layer
// budgets of GateSight (Sec. 4.2, Appendix G: every head of layer l keeps its
// prompt plus K_l entries), and the shared list of a layer (Appendix H: one
// list per layer ranked by the larger of its per-head scores).
//
// One workgroup per list: 128 threads (2 waves) when the n - prot candidate
// keys fit LDS next to the select state, else 1024 threads with the keys in
// dynamic LDS or, past that, read again on every pass.  The keys (rank_key of
// the score, or the draw's 24-bit integer) are staged in LDS, then the radix
// select and the chronological emit of select_lds.hpp write the kept indices
// in increasing order, ties at the threshold to the lowest positions.
#include "kvevict_device.hpp"
#include "kvevict_launch.hpp"
#include "select_lds.hpp"

namespace kvevict {
namespace {

constexpr int kThreads = kSelectThreads;
// The top-K of lists that fit LDS, drawn or stored: 128 threads, so twice as
// many lists are in flight per CU as with 256 (same-process A/B, keep sets
// identical: random draw batch 154 -> 125 us, paged 93 -> 78 us, the 30-round
// shape 322 -> 288 us; stored scores KeyDiff 154 -> 129 us, shared max over
// heads 25 -> 21 us, paged in place 93 -> 90 us).
constexpr int kShortThreads = 128;
constexpr int kBigThreads = 1024;           // workgroup for lists longer than kMaxLdsKeys
constexpr int32_t kMaxLdsKeys = 15360;      // 60 KiB of keys (+ ~1 KiB static LDS)
constexpr int32_t kMaxBigLdsKeys = 38848;   // 151.75 KiB of keys + the 8.2 KiB select state: 160 KiB

struct TopkArgs {
  int32_t* kept_idx;
  int64_t kept_ld;
  int32_t* kept_count;  // optional: prot + kept candidates of each list
  const float* scores;
  int64_t ld;
  int32_t n, K, prot;
  int32_t L, H;                       // L > 0: list (g, h) = g*H + h keeps kk[g % L]
  int32_t kk[kMaxBudgetLayers];       // candidates kept per head in each layer
};

template <bool kKeysInLds, int NT>
__global__ __launch_bounds__(NT) void select_topk_kernel(TopkArgs a) {
  int32_t* __restrict__ kept_idx = a.kept_idx;
  const float* __restrict__ scores = a.scores;
  const int64_t kept_ld = a.kept_ld, ld = a.ld;
  const int32_t n = a.n, prot = a.prot;
  extern __shared__ uint32_t s_keys[];
  __shared__ SelectShared<NT> sh;

  const int64_t list = blockIdx.x;
  const float* row = scores + list * ld;
  int32_t* out = kept_idx + list * kept_ld;
  const int32_t m = n - prot;  // candidates
  const int32_t kk = a.L > 0 ? a.kk[(list / a.H) % a.L] : a.K - prot;  // candidates to keep
  const int tid = threadIdx.x;

  for (int32_t j = tid; j < prot; j += NT) out[j] = j;
  if (a.kept_count && tid == 0) a.kept_count[list] = prot + kk;
  if (kk <= 0) return;

  if (kKeysInLds) {
    for (int32_t i = tid; i < m; i += NT) s_keys[i] = rank_key(row[prot + i]);
    __syncthreads();
  }
  auto key_at = [&](int32_t i) -> uint32_t {
    return kKeysInLds ? s_keys[i] : rank_key(row[prot + i]);
  };

  uint32_t thr = 0u, need_eq = 0xffffffffu;  // kk == m: keep every candidate
  if (kk < m) radix_select(key_at, m, kk, sh, thr, need_eq);
  emit_kept(key_at, m, thr, need_eq, sh,
            [&](uint32_t slot, int32_t i) { out[prot + slot] = prot + i; });
}

// True if a list of m keys fits the big kernel's dynamic LDS on the current
// device (gfx950: 160 KiB per workgroup), after raising the kernel's limit.
bool big_lds_ok(int32_t m, const void* kernel) {
  if (m > kMaxBigLdsKeys) return false;
  int dev = 0, limit = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&limit, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    return false;
  const size_t need = (size_t)m * sizeof(uint32_t) + sizeof(SelectShared<kBigThreads>);
  if (need > (size_t)limit) return false;
  return hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)(m * sizeof(uint32_t))) == hipSuccess;
}

}  // namespace

hipError_t launch_select_topk(int32_t* kept_idx, int64_t kept_ld, int32_t* kept_count,
                              const float* scores, int64_t ld, int64_t num_lists, int32_t n,
                              int32_t K, int32_t prot, int32_t L, int32_t H,
                              const int32_t* layer_kk, hipStream_t stream) {
  if (num_lists == 0) return hipSuccess;
  TopkArgs a;
  a.kept_idx = kept_idx;
  a.kept_ld = kept_ld;
  a.kept_count = kept_count;
  a.scores = scores;
  a.ld = ld;
  a.n = n;
  a.K = K;
  a.prot = prot;
  a.L = layer_kk ? L : 0;
  a.H = H;
  for (int32_t l = 0; l < kMaxBudgetLayers; ++l) a.kk[l] = (layer_kk && l < L) ? layer_kk[l] : 0;
  const int32_t m = n - prot;
  if (num_lists > max_workgroups(m <= kMaxLdsKeys ? kShortThreads : kBigThreads))
    return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)num_lists);
  if (m <= kMaxLdsKeys) {
    const size_t lds = (size_t)(m > 0 ? m : 1) * sizeof(uint32_t);
    hipLaunchKernelGGL((select_topk_kernel<true, kShortThreads>), grid, dim3(kShortThreads), lds,
                       stream, a);
  } else if (big_lds_ok(m, reinterpret_cast<const void*>(&select_topk_kernel<true, kBigThreads>))) {
    hipLaunchKernelGGL((select_topk_kernel<true, kBigThreads>), grid, dim3(kBigThreads),
                       (size_t)m * sizeof(uint32_t), stream, a);
  } else {
    hipLaunchKernelGGL((select_topk_kernel<false, kBigThreads>), grid, dim3(kBigThreads), 0,
                       stream, a);
  }
  return hipGetLastError();
}

namespace {

struct DrawArgs {
  int32_t* kept_idx;
  int64_t kept_ld;
  int32_t L, H, n, K, prot, shared_draw;
  uint64_t seed;
  uint32_t round;
};

// The random scorer and the per-list top-K in one launch: list `blockIdx.x`
// draws its candidates' Philox scores (the stream of kvevict_score_random) as
// their 24-bit integers (draw_key: the same order as the scores) straight into
// LDS, or, for lists longer than LDS holds, draws them again on every pass; no
// score buffer is written or read.  The select then takes three radix passes
// over uniformly filled digits.
template <bool kKeysInLds, int NT>
__global__ __launch_bounds__(NT) void draw_select_kernel(DrawArgs a) {
  extern __shared__ uint32_t s_keys[];
  __shared__ SelectShared<NT> sh;
  const int64_t list = blockIdx.x;
  const int32_t n = a.n, prot = a.prot, m = n - prot, kk = a.K - prot;
  int32_t* out = a.kept_idx + list * a.kept_ld;
  const int tid = threadIdx.x;
  uint64_t request, layer, head;
  if (a.shared_draw) {
    request = (uint64_t)(list / a.L);
    layer = (uint64_t)(list % a.L);
    head = 0;
  } else {
    const int64_t lh = (int64_t)a.L * a.H;
    request = (uint64_t)(list / lh);
    layer = (uint64_t)((list / a.H) % a.L);
    head = (uint64_t)(list % a.H);
  }
  const uint64_t ctr2 = (request << 32) | a.round;

  for (int32_t j = tid; j < prot; j += NT) out[j] = j;
  if (kk <= 0) return;
  if (kKeysInLds) {
    for (int32_t c = prot / 4 + tid; 4 * c < n; c += NT) {
      const Philox4x64 r = philox4x64_10((uint64_t)c, head, layer, ctr2, a.seed, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int32_t i = 4 * c + q;
        if (i >= prot && i < n) s_keys[i - prot] = draw_key(r.w[q]);
      }
    }
    __syncthreads();
  }
  auto key_at = [&](int32_t i) -> uint32_t {
    if (kKeysInLds) return s_keys[i];
    const int32_t slot = prot + i;
    const Philox4x64 r = philox4x64_10((uint64_t)(slot >> 2), head, layer, ctr2, a.seed, 0);
    // word slot % 4, chosen with constant indices (a variable index would place r in memory)
    const uint64_t w = (slot & 2) ? ((slot & 1) ? r.w[3] : r.w[2]) : ((slot & 1) ? r.w[1] : r.w[0]);
    return draw_key(w);
  };
  uint32_t thr = 0u, need_eq = 0xffffffffu;  // kk == m: keep every candidate
  if (kk < m) radix_select<24>(key_at, m, kk, sh, thr, need_eq);
  emit_kept(key_at, m, thr, need_eq, sh,
            [&](uint32_t slot, int32_t i) { out[prot + slot] = prot + i; });
}

// Shared score of each (group, position): the score of the head whose
// rank_key is largest, the lowest head among equals (its bits are kept).
__global__ __launch_bounds__(kThreads) void reduce_max_heads_kernel(
    float* __restrict__ out, int64_t out_ld, const float* __restrict__ scores, int64_t ld,
    int64_t g0, int32_t H, int32_t n) {
  const int64_t g = g0 + blockIdx.y;
  const int32_t i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  const float* base = scores + g * H * ld + i;
  float best = base[0];
  uint32_t best_key = rank_key(best);
  for (int32_t h = 1; h < H; ++h) {
    const float v = base[h * ld];
    const uint32_t k = rank_key(v);
    if (k > best_key) {
      best = v;
      best_key = k;
    }
  }
  out[g * out_ld + i] = best;
}

}  // namespace

hipError_t launch_draw_select(int32_t* kept_idx, int64_t kept_ld, int64_t num_lists, int32_t L,
                              int32_t H, int32_t n, int32_t K, int32_t prot, uint64_t seed,
                              uint32_t round, bool shared_draw, hipStream_t stream) {
  if (num_lists == 0) return hipSuccess;
  DrawArgs a;
  a.kept_idx = kept_idx;
  a.kept_ld = kept_ld;
  a.L = L;
  a.H = H;
  a.n = n;
  a.K = K;
  a.prot = prot;
  a.shared_draw = shared_draw ? 1 : 0;
  a.seed = seed;
  a.round = round;
  const int32_t m = n - prot;
  if (num_lists > max_workgroups(m <= kMaxLdsKeys ? kShortThreads : kBigThreads))
    return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)num_lists);
  if (m <= kMaxLdsKeys) {
    const size_t lds = (size_t)(m > 0 ? m : 1) * sizeof(uint32_t);
    hipLaunchKernelGGL((draw_select_kernel<true, kShortThreads>), grid, dim3(kShortThreads), lds,
                       stream, a);
  } else if (big_lds_ok(m, reinterpret_cast<const void*>(&draw_select_kernel<true, kBigThreads>))) {
    hipLaunchKernelGGL((draw_select_kernel<true, kBigThreads>), grid, dim3(kBigThreads),
                       (size_t)m * sizeof(uint32_t), stream, a);
  } else {
    hipLaunchKernelGGL((draw_select_kernel<false, kBigThreads>), grid, dim3(kBigThreads), 0,
                       stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_reduce_max_heads(float* out, int64_t out_ld, const float* scores, int64_t ld,
                                   int64_t num_groups, int32_t H, int32_t n, hipStream_t stream) {
  if (num_groups == 0 || n == 0) return hipSuccess;
  const unsigned bx = (unsigned)((n + kThreads - 1) / kThreads);
  const int64_t kMaxY = 65535;
  for (int64_t g0 = 0; g0 < num_groups; g0 += kMaxY) {
    const int64_t rows = (num_groups - g0 < kMaxY) ? num_groups - g0 : kMaxY;
    hipLaunchKernelGGL(reduce_max_heads_kernel, dim3(bx, (unsigned)rows), dim3(kThreads), 0,
                       stream, out, out_ld, scores, ld, g0, H, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kvevict
