// Top-k of a list of 32-bit rank keys held by one workgroup of NT threads
// (NT a multiple of 64, at least 256)
// ("Random Attention" blog summary, Algorithm 1: top-K per KV head; ties go to
// the lower position).
//
// radix_select finds the threshold key T and how many keys equal to T are
// kept with an 8-bit-digit radix select (at most 4 histogram passes, stopping
// as soon as the chosen bucket is taken whole).  emit_kept then visits the kept
// keys in increasing position with wave ballots and mbcnt prefix counts: a
// kept key's output slot is the number of kept keys before it, so the keys
// equal to T that are kept are the lowest positions.
#pragma once

#include "kvevict_device.hpp"

namespace kvevict {

constexpr int kSelectThreads = 256;

template <int NT = kSelectThreads>
struct SelectShared {
  static_assert(NT % kWave == 0 && NT >= 256, "one thread per histogram bin");
  uint32_t hist[256];
  uint32_t scan[NT / kWave];
  uint32_t pick[3];
  uint32_t tile[2 * (NT / kWave)];
};

// Keep kk of the m keys key_at(0..m-1), 0 < kk < m: every key > thr, and the
// first need_eq keys == thr (need_eq = 0xffffffff: every key == thr).
template <int NT, class KeyAt>
__device__ void radix_select(KeyAt key_at, int32_t m, int32_t kk, SelectShared<NT>& sh,
                             uint32_t& thr, uint32_t& need_eq) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0u, mask = 0u, remaining = (uint32_t)kk;
  bool whole_bucket = false;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) sh.hist[tid] = 0u;
    __syncthreads();
    for (int32_t i = tid; i < m; i += NT) {
      const uint32_t k = key_at(i);
      if ((k & mask) == prefix) atomicAdd(&sh.hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    // thread t < 256 holds bin 255 - t (the others count 0), so the inclusive scan
    // counts keys in bins >= 255 - t
    const uint32_t c = tid < 256 ? sh.hist[255 - tid] : 0u;
    uint32_t total;
    const uint32_t incl = block_inclusive_scan<NT>(c, sh.scan, &total);
    const uint32_t excl = incl - c;
    if (excl < remaining && incl >= remaining) {
      sh.pick[0] = 255u - (uint32_t)tid;
      sh.pick[1] = remaining - excl;
      sh.pick[2] = c;
    }
    __syncthreads();
    const uint32_t digit = sh.pick[0];
    const uint32_t cnt = sh.pick[2];
    remaining = sh.pick[1];
    prefix |= digit << shift;
    mask |= 0xffu << shift;
    __syncthreads();
    if (remaining == cnt) {  // the whole bucket is kept: keep every key >= prefix
      whole_bucket = true;
      break;
    }
  }
  thr = prefix;
  need_eq = whole_bucket ? 0xffffffffu : remaining;
}

// Calls out(slot, i) for every kept key i (key > thr, or == thr among the
// first need_eq such), slot = number of kept keys before position i.
template <int NT, class KeyAt, class Out>
__device__ void emit_kept(KeyAt key_at, int32_t m, uint32_t thr, uint32_t need_eq,
                          SelectShared<NT>& sh, Out out) {
  constexpr int kWaves = NT / kWave;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  uint32_t carry_gt = 0u, carry_eq = 0u;
  for (int32_t base = 0; base < m; base += NT) {
    const int32_t i = base + tid;
    const bool valid = i < m;
    const uint32_t k = valid ? key_at(i) : 0u;
    const bool gt = valid && k > thr;
    const bool eq = valid && k == thr;
    const uint64_t bg = __ballot(gt);
    const uint64_t be = __ballot(eq);
    if (lane_id() == 0) {
      sh.tile[wave] = (uint32_t)__popcll(bg);
      sh.tile[kWaves + wave] = (uint32_t)__popcll(be);
    }
    __syncthreads();
    uint32_t pre_gt = 0u, pre_eq = 0u, tot_gt = 0u, tot_eq = 0u;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t g = sh.tile[w], e = sh.tile[kWaves + w];
      pre_gt += (w < wave) ? g : 0u;
      pre_eq += (w < wave) ? e : 0u;
      tot_gt += g;
      tot_eq += e;
    }
    __syncthreads();
    const uint32_t gt_before = carry_gt + pre_gt + count_below(bg);
    const uint32_t eq_before = carry_eq + pre_eq + count_below(be);
    if (gt || (eq && eq_before < need_eq)) out(gt_before + min(eq_before, need_eq), i);
    carry_gt += tot_gt;
    carry_eq += tot_eq;
  }
}

}  // namespace kvevict
