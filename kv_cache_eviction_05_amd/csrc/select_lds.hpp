// Top-k of a list of 32-bit rank keys held by one workgroup of NT threads
// (NT a multiple of 64, at least 128: one or two histogram bins per thread)
// ("Random Attention" blog summary, Algorithm 1: top-K per KV head; ties go to
// the lower position).
//
// radix_select finds the threshold key T and how many keys equal to T are
// kept with a radix select that stops as soon as the chosen bucket is taken
// whole: 8-bit digits (at most 4 passes) for NT < 1024, and 11/11/10-bit
// digits (at most 3 passes) for the 1024-thread workgroups of long lists.  The
// top digit of a float key is its sign and exponent, which few values share:
// the wider digit spreads a long list's LDS atomics over more bins (64 lists
// of 32,512 keys: 57 us against 69 us).  The short lists of 256-thread
// workgroups lose with it (more bins to clear and scan per key), so they keep
// 8-bit digits.  emit_kept then visits the kept
// keys in increasing position with wave ballots and mbcnt prefix counts: a
// kept key's output slot is the number of kept keys before it, so the keys
// equal to T that are kept are the lowest positions.
#pragma once

#include "kvevict_device.hpp"

namespace kvevict {

constexpr int kSelectThreads = 256;

// Digit width of radix pass p for a workgroup of NT threads.
// Keys of kKeyBits = 24 (the raw draws of the random scorer) take 11/11/2 or
// 8/8/8-bit digits: three passes.
template <int NT, int kKeyBits = 32>
__host__ __device__ constexpr int select_digit_bits(int p) {
  return kKeyBits == 24 ? (NT >= 1024 ? (p < 2 ? 11 : 2) : 8)
                        : (NT >= 1024 ? (p < 2 ? 11 : 10) : 8);
}
template <int NT, int kKeyBits = 32>
__host__ __device__ constexpr int select_passes() {
  return (kKeyBits == 24 || NT >= 1024) ? 3 : 4;
}

// NT must be the workgroup size: the select's loops stride by it and its scans
// take one word per wave.
template <int NT>
struct SelectShared {
  static_assert(NT % kWave == 0 && NT >= 128, "at most two histogram bins per thread");
  static constexpr int kBins = 1 << select_digit_bits<NT>(0);
  static_assert(kBins % NT == 0 && kBins / NT <= 2, "one or two bins per thread");
  uint32_t hist[kBins];
  uint32_t scan[NT / kWave];
  uint32_t pick[3];
  uint32_t tile[2 * (NT / kWave)];
};

// Keep kk of the m keys key_at(0..m-1), 0 < kk < m: every key > thr, and the
// first need_eq keys == thr (need_eq = 0xffffffff: every key == thr).
// kKeyBits: the keys use only their low kKeyBits bits (32 or 24).
template <int kKeyBits = 32, int NT, class KeyAt>
__device__ void radix_select(KeyAt key_at, int32_t m, int32_t kk, SelectShared<NT>& sh,
                             uint32_t& thr, uint32_t& need_eq) {
  static_assert(kKeyBits == 32 || kKeyBits == 24, "32-bit rank keys or 24-bit draws");
  const int tid = threadIdx.x;
  uint32_t prefix = 0u, mask = 0u, remaining = (uint32_t)kk;
  bool whole_bucket = false;
  int shift = kKeyBits;
#pragma unroll
  for (int pass = 0; pass < select_passes<NT, kKeyBits>(); ++pass) {
    const int bits = select_digit_bits<NT, kKeyBits>(pass);
    const uint32_t bins = 1u << bits;
    shift -= bits;
    for (uint32_t b = tid; b < bins; b += NT) sh.hist[b] = 0u;
    __syncthreads();
    for (int32_t i = tid; i < m; i += NT) {
      const uint32_t k = key_at(i);
      if ((k & mask) == prefix) atomicAdd(&sh.hist[(k >> shift) & (bins - 1u)], 1u);
    }
    __syncthreads();
    // thread t holds bins [top - per, top), top = bins - per*t, highest first (with
    // fewer bins than threads, threads t < bins hold one each), so the inclusive
    // scan counts the keys in bins >= top - per
    const uint32_t per = bins >= (uint32_t)NT ? bins / NT : 1u;
    const bool holds = (uint32_t)tid * per < bins;
    const uint32_t top = holds ? bins - per * (uint32_t)tid : 0u;
    uint32_t h[2], c = 0u;
#pragma unroll
    for (uint32_t b = 0; b < 2; ++b) {
      h[b] = (holds && b < per) ? sh.hist[top - 1u - b] : 0u;
      c += h[b];
    }
    uint32_t total;
    const uint32_t incl = block_inclusive_scan<NT>(c, sh.scan, &total);
    const uint32_t excl = incl - c;
    if (excl < remaining && incl >= remaining) {
      uint32_t acc = excl;
#pragma unroll
      for (uint32_t b = 0; b < 2; ++b) {
        if (b < per && acc < remaining && acc + h[b] >= remaining) {
          sh.pick[0] = top - 1u - b;
          sh.pick[1] = remaining - acc;
          sh.pick[2] = h[b];
        }
        acc += h[b];
      }
    }
    __syncthreads();
    const uint32_t digit = sh.pick[0];
    const uint32_t cnt = sh.pick[2];
    remaining = sh.pick[1];
    prefix |= digit << shift;
    mask |= (bins - 1u) << shift;
    __syncthreads();
    if (remaining == cnt) {  // the whole bucket is kept: keep every key >= prefix
      whole_bucket = true;
      break;
    }
  }
  thr = prefix;
  need_eq = whole_bucket ? 0xffffffffu : remaining;
}

// emit_kept for short lists (NT < 1024): one ballot round of NT keys at a
// time, with two barriers per round.
template <int NT, class KeyAt, class Out>
__device__ void emit_kept_rounds(KeyAt key_at, int32_t m, uint32_t thr, uint32_t need_eq,
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

// Calls out(slot, i) for every kept key i (key > thr, or == thr among the
// first need_eq such), slot = number of kept keys before position i.  Keys are
// visited in groups of kEmitRounds rounds of NT positions: every wave ballots
// its keys of the whole group first, one wave scans the per-(round, wave)
// counts, then every kept key takes its scanned prefix plus the set lanes
// below it, two barriers per group.  The scan reuses the histogram and pick
// words of `sh`, which the select no longer needs.  Long lists only (NT >=
// 1024: layers select, 64 lists of 32,512 keys, 33 us against 58 us); the
// 128- and 256-thread workgroups of short lists keep one round at a time,
// which was 5-6% faster for them.
template <int NT, class KeyAt, class Out>
__device__ void emit_kept(KeyAt key_at, int32_t m, uint32_t thr, uint32_t need_eq,
                          SelectShared<NT>& sh, Out out) {
  if constexpr (NT < 1024) {
    emit_kept_rounds<NT>(key_at, m, thr, need_eq, sh, out);
  } else {
  constexpr int kW = NT / kWave;
  constexpr int kRounds = 8;                  // rounds of NT keys per group
  constexpr int kS = kRounds * kW;            // (round, wave) slots per kind
  constexpr int kPer = 2 * kS / kWave;        // counts per lane in the scan
  static_assert(kS % (kWave / 2) == 0 && 4 * kS <= SelectShared<NT>::kBins,
                "the scan splits over the lanes; counts and prefixes fit the histogram");
  uint32_t* cnt = sh.hist;                    // [gt: kS][eq: kS]
  uint32_t* pre = sh.hist + 2 * kS;           // exclusive prefixes, same layout
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const uint32_t lane = lane_id();
  uint32_t carry_gt = 0u, carry_eq = 0u;
  for (int32_t base = 0; base < m; base += kRounds * NT) {
    uint64_t bg[kRounds], be[kRounds];
#pragma unroll
    for (int c = 0; c < kRounds; ++c) {
      const int32_t i = base + c * NT + tid;
      const bool valid = i < m;
      const uint32_t k = valid ? key_at(i) : 0u;
      bg[c] = __ballot(valid && k > thr);
      be[c] = __ballot(valid && k == thr);
      if (lane == 0) {
        cnt[c * kW + wave] = (uint32_t)__popcll(bg[c]);
        cnt[kS + c * kW + wave] = (uint32_t)__popcll(be[c]);
      }
    }
    __syncthreads();
    if (wave == 0) {  // lanes [0, 32) scan the gt counts, [32, 64) the eq counts
      uint32_t v[kPer], run = 0u;
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        v[q] = cnt[lane * kPer + q];
        run += v[q];
      }
      uint32_t incl = run;
#pragma unroll
      for (int d = 1; d < kWave / 2; d <<= 1) {
        const uint32_t t = __shfl_up(incl, d, kWave / 2);
        if ((lane & (kWave / 2 - 1)) >= (uint32_t)d) incl += t;
      }
      uint32_t p = incl - run;
#pragma unroll
      for (int q = 0; q < kPer; ++q) {
        pre[lane * kPer + q] = p;
        p += v[q];
      }
      if ((lane & (kWave / 2 - 1)) == kWave / 2 - 1) sh.pick[lane / (kWave / 2)] = incl;  // totals
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kRounds; ++c) {
      const int32_t i = base + c * NT + tid;
      const bool gt = (bg[c] >> lane) & 1u;
      const bool eq = (be[c] >> lane) & 1u;
      const uint32_t gt_before = carry_gt + pre[c * kW + wave] + count_below(bg[c]);
      const uint32_t eq_before = carry_eq + pre[kS + c * kW + wave] + count_below(be[c]);
      if (gt || (eq && eq_before < need_eq)) out(gt_before + min(eq_before, need_eq), i);
    }
    carry_gt += sh.pick[0];
    carry_eq += sh.pick[1];
  }
  }
}

}  // namespace kvevict
