// Device-side building blocks shared by the gfx950 kernels of the eviction round.
//
// Everything here is written for CDNA4 wave64: ballots are 64-bit masks,
// lane prefix counts use the mbcnt pair, block scans combine a wave-level
// shuffle scan with one LDS word per wave.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvevict {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Ranking key.  Maps an fp32 score to a uint32 whose unsigned order is the
// ranking order: larger key = better entry.  NaN ranks as -inf and -0 as +0
// (the tie between equal keys is broken by position by the callers).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t rank_key(float f) {
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) > 0x7f800000u) b = 0xff800000u;  // NaN -> -inf
  if (b == 0x80000000u) b = 0u;                           // -0 -> +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// ---------------------------------------------------------------------------
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC 2011): ten rounds of two
// 64x64->128 products; key bumped by the Weyl constants between rounds.
// ---------------------------------------------------------------------------
struct Philox4x64 {
  uint64_t w[4];
};

__device__ __forceinline__ Philox4x64 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2,
                                                   uint64_t c3, uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t lo0 = M0 * c0, hi0 = __umul64hi(M0, c0);
    const uint64_t lo1 = M1 * c2, hi1 = __umul64hi(M1, c2);
    const uint64_t n0 = hi1 ^ c1 ^ k0;
    const uint64_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
    k0 += W0;
    k1 += W1;
  }
  Philox4x64 out;
  out.w[0] = c0;
  out.w[1] = c1;
  out.w[2] = c2;
  out.w[3] = c3;
  return out;
}

// 24 random bits scaled to [0, 1); exact in fp32.
__device__ __forceinline__ float unit_from_word(uint64_t word) {
  return (float)(uint32_t)(word >> 40) * (1.0f / 16777216.0f);
}

// The same 24 bits as a rank key: unit_from_word(word) is this integer times
// 2^-24 exactly, so the two order draws alike, ties included.  The integer
// spreads uniformly over its radix digits, where a float's top byte (sign and
// exponent) piles most of [0, 1) into two or three bins.
__device__ __forceinline__ uint32_t draw_key(uint64_t word) { return (uint32_t)(word >> 40); }

// ---------------------------------------------------------------------------
// Wave / block helpers (wave64).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

// Number of set bits of `mask` in lanes below the calling lane.
__device__ __forceinline__ uint32_t count_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  const uint32_t lane = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    uint32_t t = __shfl_up(v, d, kWave);
    if (lane >= (uint32_t)d) v += t;
  }
  return v;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
  for (int d = kWave / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

// Inclusive prefix sum over a block of NT threads (NT a multiple of 64).
// `scratch` holds NT/64 words; returns the scan value and the block total.
template <int NT>
__device__ __forceinline__ uint32_t block_inclusive_scan(uint32_t v, uint32_t* scratch,
                                                         uint32_t* total) {
  constexpr int NW = NT / kWave;
  const int wave = threadIdx.x / kWave;
  uint32_t incl = wave_inclusive_scan(v);
  if (lane_id() == kWave - 1) scratch[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    uint32_t s = scratch[w];
    before += (w < wave) ? s : 0u;
    all += s;
  }
  __syncthreads();
  *total = all;
  return incl + before;
}

template <int NT>
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* scratch) {
  constexpr int NW = NT / kWave;
  const int wave = threadIdx.x / kWave;
  uint32_t s = wave_sum(v);
  if (lane_id() == 0) scratch[wave] = s;
  __syncthreads();
  uint32_t all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) all += scratch[w];
  __syncthreads();
  return all;
}

}  // namespace kvevict
