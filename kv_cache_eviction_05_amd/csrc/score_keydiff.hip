// KeyDiff key scores (GateSight Sec. 5.1, baselines paragraph): each cached
// key is scored by minus its cosine to the mean of its head's keys, taken
// without normalising the keys first, so that a per-head top-K keeps the keys
// that point away from the mean.
//
//   score[list][i] = -cos(k_i, mean_j k_j)   (mean over all n keys of the list),
//   +inf for i < prot; a zero norm gives cos = 0; zero is written as +0.
//
// The mean needs every key before any cosine.  One workgroup of 512 threads
// per list, two per CU: a row of D bf16 is VPR = D/8 16-byte vectors, thread t
// owns vector column t % VPR of rows t / VPR + k * (512 / VPR); its first 10
// such rows (11 at D = 128) stay in registers and the next 9 (D <= 128), 8 or 7
// in LDS, which at D = 128 holds 640 of 1088 rows between the two passes.  The
// other rows are read a second time soon after the first, and those reads
// mostly hit the Infinity Cache: measured on the 36,864-list batch, a plain
// read of every row once and of the streamed rows again takes 1.22x the time
// of one read; twelve register rows gained nothing, and one 1024-thread
// workgroup per CU holding 1024 rows (1.04x the bytes) was 14% slower, since
// two workgroups per CU let one list's reads overlap the other's arithmetic.
// Pass 1 accumulates the column sums in binary64 in a fixed order (lanes of a
// column with shuffles, then the waves in a tree through LDS) into the mean
// and its squared norm.  Pass 2 forms each row's dot product with the mean and
// its squared norm in binary64 and adds the VPR partials of a row with DPP lane
// moves; the binary64 work bounds the kernel as much as the reads do, so the
// lanes of a group collect VPR rows' sums before the square root and division,
// which then run once per row (not once per lane group).  At D = 128 in a
// contiguous store two rows go through the lane reduction together (one
// exchange, then three levels that serve both), and the streamed rows come
// through buffer loads from a per-step base, whose range check reads rows past
// n as zeros (no per-row bounds checks).  The result
// -dot / (sqrt(|k|^2) * sqrt(|mean|^2)) is rounded once to fp32, with IEEE
// binary64 square roots and division.  The sums run in another order than a
// plain loop's, so the binary64 cosine may differ from it by a few units of
// 2^-53 times (D + n * |sum of |k_i|| / |sum of k_i|); the fp32 score then
// equals the plain loop's rounding except where that cosine lies within this
// bound of a midpoint between two fp32 values, where it may be the other
// neighbour (one fp32 ulp away).
//
// Lists of at most 1088 keys at D = 128 in a contiguous store take a second kernel
// (score_keydiff_resident_kernel, below) that holds the whole list on chip at two waves
// per SIMD and so reads every key once: 2.00-2.03 ms against 2.10-2.15 ms on the batch
// in a same-process A/B, bit-identical scores.  It is bound by binary64 issue as much as
// by the reads (about 65% VALU busy, 20% of wave time waiting on memory); requesting the
// next list's rows behind pass 2, in a persistent form, measured the same.
#include <cmath>

#include "kvevict_device.hpp"
#include "kvevict_launch.hpp"

namespace kvevict {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kReg0 = 10;   // rows per thread held in registers
constexpr int kUnroll = 8;  // rows per thread in flight for the streamed tail

// rows per thread held in LDS: 8 KB each, next to 4*D + D doubles of sums, so that
// two workgroups fit the 160 KB of a CU
template <int VPR>
constexpr int lds_rows() { return VPR >= 64 ? 7 : VPR >= 32 ? 8 : 9; }

typedef uint32_t vec4u __attribute__((ext_vector_type(4)));

struct KeydiffArgs {
  float* scores;
  int64_t ld;
  StoreView keys;
  const vec4u* k;
  int32_t H, n, prot, vpr;
};

// Vector offset of row t < n of list (g, h), or -1 if its page id falls
// outside the pool (such a row reads as zeros).
template <bool kPaged>
__device__ __forceinline__ int64_t key_row(const KeydiffArgs& a, int64_t list, int32_t t,
                                           int32_t vpr) {
  if (!kPaged) return list * a.keys.list_stride_v + (int64_t)t * vpr;
  const int64_t g = list / a.H;
  const int32_t h = (int32_t)(list - g * a.H);
  const int32_t page = a.keys.page_table[g * a.keys.pt_ld + (t >> a.keys.page_shift)];
  if (page < 0 || (int64_t)page >= a.keys.capacity) return -1;
  const int64_t slot = ((int64_t)page << a.keys.page_shift) + (t & ((1 << a.keys.page_shift) - 1));
  return (slot * a.H + h) * vpr;
}

template <bool kPaged>
__device__ __forceinline__ vec4u load_key(const KeydiffArgs& a, int64_t list, int32_t t,
                                          int32_t vpr, int32_t col) {
  const int64_t off = key_row<kPaged>(a, list, t, vpr);
  return off >= 0 ? a.k[off + col] : vec4u{0u, 0u, 0u, 0u};
}

// Vector `col` of row t of a list, or zeros for t >= n; contiguous rows are
// addressed from the list's (uniform) base with a 32-bit offset and read
// without a branch (a row past n reads row n - 1, n >= 1, then is zeroed).
template <int VPR, bool kPaged>
__device__ __forceinline__ vec4u load_row(const KeydiffArgs& a, const vec4u* __restrict__ lb,
                                          int64_t list, int32_t t, int32_t n, int32_t col) {
  if (kPaged) return (t < n) ? load_key<true>(a, list, t, VPR, col) : vec4u{0u, 0u, 0u, 0u};
  const int32_t tt = t < n ? t : n - 1;
  const vec4u v = lb[tt * VPR + col];
  return t < n ? v : vec4u{0u, 0u, 0u, 0u};
}

// The eight bf16 of a 16-byte vector as binary64 (exact).
__device__ __forceinline__ void unpack8(vec4u v, double* x) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    x[2 * q] = (double)__uint_as_float(v[q] << 16);
    x[2 * q + 1] = (double)__uint_as_float(v[q] & 0xffff0000u);
  }
}

// Sum of a binary64 value over aligned groups of W consecutive lanes (W a power
// of two <= 64), every lane of a group receiving the sum: DPP moves within the
// 16-lane rows (pair swap, quad swap, half-row mirror, row mirror), lane
// shuffles across rows.
template <int W>
__device__ __forceinline__ double group_sum(double v) {
  auto dpp = [](double x, int ctrl) -> double {
    const uint64_t b = __double_as_longlong(x);
    const int lo = (int)(uint32_t)b, hi = (int)(uint32_t)(b >> 32);
    int rlo, rhi;
    switch (ctrl) {  // the DPP control must be a constant; every lane's source is valid
      case 0: rlo = __builtin_amdgcn_mov_dpp(lo, 0xB1, 0xF, 0xF, true);
              rhi = __builtin_amdgcn_mov_dpp(hi, 0xB1, 0xF, 0xF, true); break;
      case 1: rlo = __builtin_amdgcn_mov_dpp(lo, 0x4E, 0xF, 0xF, true);
              rhi = __builtin_amdgcn_mov_dpp(hi, 0x4E, 0xF, 0xF, true); break;
      case 2: rlo = __builtin_amdgcn_mov_dpp(lo, 0x141, 0xF, 0xF, true);
              rhi = __builtin_amdgcn_mov_dpp(hi, 0x141, 0xF, 0xF, true); break;
      default: rlo = __builtin_amdgcn_mov_dpp(lo, 0x140, 0xF, 0xF, true);
               rhi = __builtin_amdgcn_mov_dpp(hi, 0x140, 0xF, 0xF, true); break;
    }
    return __longlong_as_double((int64_t)(((uint64_t)(uint32_t)rhi << 32) | (uint32_t)rlo));
  };
  if (W >= 2) v += dpp(v, 0);   // lanes 2i <-> 2i+1
  if (W >= 4) v += dpp(v, 1);   // lanes i <-> i^2 within a quad
  if (W >= 8) v += dpp(v, 2);   // lane i <-> 7-i within 8 lanes: quad 0 <-> quad 1
  if (W >= 16) v += dpp(v, 3);  // lane i <-> 15-i within 16 lanes: half 0 <-> half 1
  if (W >= 32) v += __shfl_xor(v, 16, kWave);
  if (W >= 64) v += __shfl_xor(v, 32, kWave);
  return v;
}

// A binary64 DPP move (each half separately), every lane's source valid.
template <int kCtrl>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t b = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)b, kCtrl, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), kCtrl, 0xF, 0xF, true);
  return __longlong_as_double((int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}

// The sums of two rows' partials over each aligned group of 16 lanes, the first row's
// in the even lanes and the second's in the odd ones: even lanes swap their second-row
// partial for the odd neighbour's first-row one (lanes i, i^1), then the lanes of one
// parity add within quads (i, i^2) and across quads by rotations of 4 and 8 within the
// 16-lane row, which keep the parity.
__device__ __forceinline__ double pair_sum16(double a, double b, bool odd) {
  const double send = odd ? a : b;
  double v = (odd ? b : a) + dpp_f64<0xB1>(send);  // quad_perm [1,0,3,2]
  v += dpp_f64<0x4E>(v);                           // quad_perm [2,3,0,1]
  v += dpp_f64<0x124>(v);                          // row_ror:4
  v += dpp_f64<0x128>(v);                          // row_ror:8
  return v;
}

typedef __amdgpu_buffer_rsrc_t buf_rsrc;
// A raw buffer over `bytes` bytes from p: loads at or past the end read as zeros.  Stride 0
// makes the record count a byte count; the last word's 0x00020000 sets the data format
// field to 32-bit elements, with no swizzle and no added thread id (the raw-buffer setting
// of this GPU family).
__device__ __forceinline__ buf_rsrc rows_rsrc(const void* p, int64_t bytes) {
  const int32_t nb = bytes > 0 ? (bytes < 0x7fffffff ? (int32_t)bytes : 0x7fffffff) : 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, nb, 0x00020000);
}

// Partial dot with the mean and squared norm of one 16-byte vector.
__device__ __forceinline__ void dot_norm(vec4u v, const double* mu, double& dot, double& kk) {
  double x[8];
  unpack8(v, x);
  dot = 0.0;
  kk = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    dot = fma(x[e], mu[e], dot);
    kk = fma(x[e], x[e], kk);
  }
}

template <int VPR, bool kPaged, bool kPairOk>
__global__ __launch_bounds__(kThreads) void score_keydiff_kernel(KeydiffArgs a) {
  constexpr int32_t rpi = kThreads / VPR;  // rows per iteration
  constexpr int32_t D = VPR * 8;
  // D = 128 in a contiguous store: rows two at a time through pass 2, the streamed
  // rows through buffer loads (rows past n read as zeros)
  constexpr bool kPair = VPR == 16 && !kPaged && kPairOk;
  constexpr int kLds = lds_rows<VPR>();
  constexpr int kReg = kPair ? 11 : kReg0;
  static_assert(!kPair || (kReg + kLds) % 2 == 0, "pairs of on-chip steps");
  constexpr int32_t kCap = (kReg + kLds) * rpi;  // rows held on chip
  __shared__ vec4u s_keys[kLds][kThreads];
  __shared__ double s_part[kWaves / 2][D];   // column sums of the upper half of the waves
  __shared__ double s_mean[D];
  __shared__ double s_mm;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int32_t col = tid % VPR, r0 = tid / VPR;
  const int64_t list = blockIdx.x;
  const int32_t n = a.n;
  float* out = a.scores + list * a.ld;
  if (a.prot >= n) {  // every slot protected
    for (int32_t i = tid; i < n; i += kThreads) out[i] = INFINITY;
    return;
  }
  const vec4u* __restrict__ lb = kPaged ? a.k : a.k + list * a.keys.list_stride_v;

  // --- load the rows held on chip; pass 1: column sums ---------------------------
  vec4u reg[kReg];
#pragma unroll
  for (int k = 0; k < kReg; ++k) {
    const int32_t t = r0 + k * rpi;
    reg[k] = load_row<VPR, kPaged>(a, lb, list, t, n, col);
  }
  double sum[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sum[e] = 0.0;
  auto add = [&](vec4u v) {
    double x[8];
    unpack8(v, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) sum[e] += x[e];
  };
#pragma unroll
  for (int k0 = 0; k0 < kLds; k0 += 4) {  // staged into LDS four rows at a time
    vec4u stage[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int32_t t = r0 + (kReg + k0 + k) * rpi;
      stage[k] = (k0 + k < kLds) ? load_row<VPR, kPaged>(a, lb, list, t, n, col)
                                 : vec4u{0u, 0u, 0u, 0u};
    }
    if (k0 == 0) {
#pragma unroll
      for (int k = 0; k < kReg; ++k) add(reg[k]);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (k0 + k < kLds) {
        s_keys[k0 + k][tid] = stage[k];  // read back by this thread only
        add(stage[k]);
      }
    }
  }
  const uint32_t row_off = (uint32_t)(r0 * VPR + col) * 16u;  // this thread's vector in a step
  if constexpr (kPair) {
    // streamed tail through a buffer starting at the step's first row
    for (int32_t b0 = kCap; b0 < n; b0 += rpi * kUnroll) {
      const buf_rsrc rs = rows_rsrc(lb + (int64_t)b0 * VPR, (int64_t)(n - b0) * VPR * 16);
      vec4u v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, row_off + u * rpi * VPR * 16, 0, 0);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) add(v[u]);
    }
  }
  // streamed tail: whole steps of kUnroll rows per thread without bounds checks, then
  // the last partial step checked (the same rows in the same order either way)
  int32_t b0 = kPair ? n : kCap;
  for (; b0 + rpi * kUnroll <= n; b0 += rpi * kUnroll) {
    vec4u v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int32_t t = b0 + r0 + u * rpi;
      v[u] = kPaged ? load_key<true>(a, list, t, VPR, col) : lb[t * VPR + col];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) add(v[u]);
  }
  if (b0 < n) {
    vec4u v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = load_row<VPR, kPaged>(a, lb, list, b0 + r0 + u * rpi, n, col);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) add(v[u]);
  }
  // the lanes of one column in a wave (col, col + VPR, ...), then the waves in a tree
#pragma unroll
  for (int off = VPR; off < kWave; off <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) sum[e] += __shfl_xor(sum[e], off, kWave);
#pragma unroll
  for (int half = kWaves / 2; half >= 1; half >>= 1) {
    if (wave >= half && wave < 2 * half && lane < VPR) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_part[wave - half][col * 8 + e] = sum[e];
    }
    __syncthreads();
    if (wave < half && lane < VPR) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sum[e] += s_part[wave][col * 8 + e];
    }
    __syncthreads();
  }
  if (wave == 0) {
    double mm_part = 0.0;
    if (lane < VPR) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double mean = sum[e] / (double)n;
        s_mean[col * 8 + e] = mean;
        mm_part += mean * mean;
      }
    }
    for (int off = kWave / 2; off > 0; off >>= 1) mm_part += __shfl_xor(mm_part, off, kWave);
    if (lane == 0) s_mm = mm_part;
  }
  __syncthreads();
  const double mm = s_mm;
  const double mnorm = sqrt(mm);  // correctly rounded, as every sqrt and divide below
  // Hide the held rows' values from the compiler between the passes, so it
  // converts them again rather than keeping 64 binary64 values of pass 1 live
  // (which would spill).
#pragma unroll
  for (int k = 0; k < kReg; ++k)
#pragma unroll
    for (int q = 0; q < 4; ++q) asm volatile("" : "+v"(reg[k][q]));
  double mu[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mu[e] = s_mean[col * 8 + e];

  // --- pass 2: per-row dot with the mean and squared norm ------------------------
  if constexpr (kPair) {
    // Two steps at a time: after pair_sum16 the even lanes of a 16-lane group hold the
    // sums of the first step's row, the odd lanes the second's; lane col keeps those of
    // step kb + col, and every 16 steps (and at the end) each lane finishes its kept row.
    const bool odd = (col & 1) != 0;
    double bdot = 0.0, bkk = 0.0;
    auto keep2 = [&](int32_t k, vec4u v0, vec4u v1) __attribute__((always_inline)) {
      double d0, q0, d1, q1;
      dot_norm(v0, mu, d0, q0);
      dot_norm(v1, mu, d1, q1);
      const double d = pair_sum16(d0, d1, odd);
      const double q = pair_sum16(q0, q1, odd);
      const bool mine = (col >> 1) == ((k >> 1) & 7);
      bdot = mine ? d : bdot;
      bkk = mine ? q : bkk;
    };
    auto flush = [&](int32_t k) __attribute__((always_inline)) {  // steps k - k % 16 .. k
      const int32_t kb = k & ~15;
      const int32_t t = r0 + (kb + col) * rpi;
      if (kb + col <= k && t < n) {
        float sc = INFINITY;
        if (t >= a.prot) {
          const double den = sqrt(bkk) * mnorm;
          sc = (den > 0.0) ? (float)(-(bdot / den)) : 0.0f;
          if (sc == 0.0f) sc = 0.0f;  // -0 written as +0
        }
        out[t] = sc;
      }
    };
#pragma unroll
    for (int k = 0; k < kReg + kLds; k += 2) {
      const vec4u v0 = k < kReg ? reg[k] : s_keys[k - kReg][tid];
      const vec4u v1 = k + 1 < kReg ? reg[k + 1] : s_keys[k + 1 - kReg][tid];
      keep2(k, v0, v1);
      if (((k + 1) & 15) == 15) flush(k + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    int32_t k = kReg + kLds;
    for (int32_t c0 = kCap; c0 < n; c0 += rpi * kUnroll) {  // the streamed tail again
      const buf_rsrc rs = rows_rsrc(lb + (int64_t)c0 * VPR, (int64_t)(n - c0) * VPR * 16);
      vec4u v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, row_off + u * rpi * VPR * 16, 0, 0);
#pragma unroll
      for (int u = 0; u < kUnroll; u += 2, k += 2) {
        keep2(k, v[u], v[u + 1]);
        if (((k + 1) & 15) == 15) flush(k + 1);
      }
    }
    if ((k & 15) != 0) flush(k - 1);
    return;
  }
  // Each row's sums end in all VPR lanes of its group; lane `col` keeps those of
  // the group's row of step kb + col, and every VPR steps (and at the end) each
  // lane finishes its kept row, so the binary64 square root and division run
  // once per row rather than once per lane group.
  double bdot = 0.0, bkk = 0.0;
  auto keep = [&](int32_t k, double dot, double kk) {
    dot = group_sum<VPR>(dot);
    kk = group_sum<VPR>(kk);
    const bool mine = col == (k & (VPR - 1));
    bdot = mine ? dot : bdot;
    bkk = mine ? kk : bkk;
  };
  auto flush = [&](int32_t k) {  // steps k - k % VPR .. k are kept
    const int32_t kb = k & ~(VPR - 1);
    const int32_t t = r0 + (kb + col) * rpi;
    if (kb + col <= k && t < n) {
      float sc = INFINITY;
      if (t >= a.prot) {
        const double den = sqrt(bkk) * mnorm;
        sc = (den > 0.0) ? (float)(-(bdot / den)) : 0.0f;
        if (sc == 0.0f) sc = 0.0f;  // -0 written as +0
      }
      out[t] = sc;
    }
  };
  // one row at a time: interleaving the rows' binary64 temporaries would spill
#pragma unroll
  for (int k = 0; k < kReg; ++k) {
    double dot, kk;
    dot_norm(reg[k], mu, dot, kk);
    keep(k, dot, kk);
    if ((k & (VPR - 1)) == VPR - 1) flush(k);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int k = 0; k < kLds; ++k) {
    double dot, kk;
    dot_norm(s_keys[k][tid], mu, dot, kk);
    keep(kReg + k, dot, kk);
    if (((kReg + k) & (VPR - 1)) == VPR - 1) flush(kReg + k);
    __builtin_amdgcn_sched_barrier(0);
  }
  int32_t k = kReg + kLds;
  auto step = [&](const vec4u* v) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u, ++k) {
      double dot, kk;
      dot_norm(v[u], mu, dot, kk);
      keep(k, dot, kk);
      if ((k & (VPR - 1)) == VPR - 1) flush(k);
    }
  };
  int32_t c0 = kCap;
  for (; c0 + rpi * kUnroll <= n; c0 += rpi * kUnroll) {  // the streamed tail again
    vec4u v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int32_t t = c0 + r0 + u * rpi;
      v[u] = kPaged ? load_key<true>(a, list, t, VPR, col) : lb[t * VPR + col];
    }
    step(v);
  }
  if (c0 < n) {
    vec4u v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = load_row<VPR, kPaged>(a, lb, list, c0 + r0 + u * rpi, n, col);
    step(v);
  }
  if ((k & (VPR - 1)) != 0) flush(k - 1);
}

// Whole lists on chip: D = 128 in a contiguous store with n <= kResCap (1088) rows.
// One workgroup of 256 threads per list and two per CU (256 VGPRs per lane at two waves
// per SIMD, 78 KB of LDS each); thread t owns vector column t % 16 of rows t / 16 + 16 k,
// steps k < 49 in registers and the next 19 in LDS, so every key is read once.  The same
// arithmetic as the kernel above in its two-row form; the column sums over the 16 rows
// of a step's threads and the 4 waves run in another order, covered by the same bound.
constexpr int kResThreads = 256;
constexpr int kResWaves = kResThreads / kWave;
constexpr int kResRpi = kResThreads / 16;  // rows per step
constexpr int kResReg = 49;                // register steps per thread
constexpr int kResLds = 19;                // LDS steps per thread
constexpr int kResSteps = kResReg + kResLds;
constexpr int32_t kResCap = kResSteps * kResRpi;
static_assert(kResSteps % 2 == 0, "pairs of steps");

__global__ __launch_bounds__(kResThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void score_keydiff_resident_kernel(KeydiffArgs a) {
  constexpr int32_t D = 128;
  constexpr uint32_t kStepBytes = kResRpi * D * 2;
  __shared__ vec4u s_keys[kResLds][kResThreads];
  __shared__ double s_red[kResWaves / 2][D];  // column sums of the upper waves, then the mean
  __shared__ double s_mm;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int32_t col = tid % 16, r0 = tid / 16;
  const int64_t list = blockIdx.x;
  const int32_t n = a.n;
  float* out = a.scores + list * a.ld;
  if (a.prot >= n) {  // every slot protected
    for (int32_t i = tid; i < n; i += kResThreads) out[i] = INFINITY;
    return;
  }
  const vec4u* __restrict__ lb = a.k + list * a.keys.list_stride_v;
  const buf_rsrc rs = rows_rsrc(lb, (int64_t)n * D * 2);  // rows past n read as zeros
  const uint32_t voff = (uint32_t)tid * 16u;                // this thread's vector in a step

  // --- load every row; pass 1: column sums ------------------------------------------
  vec4u reg[kResReg];
#pragma unroll
  for (int k = 0; k < kResReg; ++k)
    reg[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, k * kStepBytes, 0);
  double sum[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sum[e] = 0.0;
  auto add = [&](vec4u v) {
    double x[8];
    unpack8(v, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) sum[e] += x[e];
  };
#pragma unroll
  for (int k0 = 0; k0 < kResLds; k0 += 4) {  // staged into LDS four rows at a time
    vec4u stage[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k0 + k < kResLds)
        stage[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, (kResReg + k0 + k) * kStepBytes, 0);
    if (k0 == 0) {
#pragma unroll
      for (int k = 0; k < kResReg; ++k) add(reg[k]);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (k0 + k < kResLds) {
        s_keys[k0 + k][tid] = stage[k];  // read back by this thread only
        add(stage[k]);
      }
    }
  }
  // the four lanes of one column in a wave, then the waves in a tree
#pragma unroll
  for (int off = 16; off < kWave; off <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) sum[e] += __shfl_xor(sum[e], off, kWave);
#pragma unroll
  for (int half = kResWaves / 2; half >= 1; half >>= 1) {
    if (wave >= half && wave < 2 * half && lane < 16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_red[wave - half][col * 8 + e] = sum[e];
    }
    __syncthreads();
    if (wave < half && lane < 16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sum[e] += s_red[wave][col * 8 + e];
    }
    __syncthreads();
  }
  if (wave == 0) {
    double mm_part = 0.0;
    if (lane < 16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double mean = sum[e] / (double)n;
        s_red[0][col * 8 + e] = mean;
        mm_part += mean * mean;
      }
    }
    for (int off = kWave / 2; off > 0; off >>= 1) mm_part += __shfl_xor(mm_part, off, kWave);
    if (lane == 0) s_mm = mm_part;
  }
  __syncthreads();
  const double mnorm = sqrt(s_mm);
#pragma unroll
  for (int k = 0; k < kResReg; ++k)
#pragma unroll
    for (int q = 0; q < 4; ++q) asm volatile("" : "+v"(reg[k][q]));
  double mu[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mu[e] = s_red[0][col * 8 + e];

  // --- pass 2: two steps at a time, as in the streaming kernel --------------------------
  // (the same lambdas as there: one shared helper struct compiled the flushes to selects
  // instead of branches, 136 more VALU instructions per wave, and measured 2% slower)
  const bool odd = (col & 1) != 0;
  double bdot = 0.0, bkk = 0.0;
  auto keep2 = [&](int32_t k, vec4u v0, vec4u v1) __attribute__((always_inline)) {
    double d0, q0, d1, q1;
    dot_norm(v0, mu, d0, q0);
    dot_norm(v1, mu, d1, q1);
    const double d = pair_sum16(d0, d1, odd);
    const double q = pair_sum16(q0, q1, odd);
    const bool mine = (col >> 1) == ((k >> 1) & 7);
    bdot = mine ? d : bdot;
    bkk = mine ? q : bkk;
  };
  auto flush = [&](int32_t k) __attribute__((always_inline)) {  // steps k - k % 16 .. k
    const int32_t kb = k & ~15;
    const int32_t t = r0 + (kb + col) * kResRpi;
    if (kb + col <= k && t < n) {
      float sc = INFINITY;
      if (t >= a.prot) {
        const double den = sqrt(bkk) * mnorm;
        sc = (den > 0.0) ? (float)(-(bdot / den)) : 0.0f;
        if (sc == 0.0f) sc = 0.0f;  // -0 written as +0
      }
      out[t] = sc;
    }
  };
#pragma unroll
  for (int k = 0; k < kResSteps; k += 2) {
    if (k * kResRpi < n) {  // the same for every thread
      const vec4u v0 = k < kResReg ? reg[k] : s_keys[k - kResReg][tid];
      const vec4u v1 = k + 1 < kResReg ? reg[k + 1] : s_keys[k + 1 - kResReg][tid];
      keep2(k, v0, v1);
    }
    if (((k + 1) & 15) == 15) flush(k + 1);
    __builtin_amdgcn_sched_barrier(0);
  }
  if ((kResSteps & 15) != 0) flush(kResSteps - 1);
}

}  // namespace

hipError_t launch_score_keydiff(float* scores, int64_t ld, const StoreView& keys, const void* k,
                                int32_t D, int32_t H, int64_t num_lists, int32_t n, int32_t prot,
                                hipStream_t stream) {
  if (num_lists == 0 || n == 0) return hipSuccess;
  if (num_lists > max_workgroups(kThreads)) return hipErrorInvalidConfiguration;
  KeydiffArgs a;
  a.scores = scores;
  a.ld = ld;
  a.keys = keys;
  a.k = static_cast<const vec4u*>(k);
  a.H = H;
  a.n = n;
  a.prot = prot;
  a.vpr = D / 8;
  const dim3 grid((unsigned)num_lists), block(kThreads);
  // buffer loads address a list's streamed rows with 32-bit byte counts
  const bool pair_ok = (int64_t)n * D * 2 <= 0x7fffffff;
  if (!keys.paged && D == 128 && n <= kResCap) {
    hipLaunchKernelGGL(score_keydiff_resident_kernel, grid, dim3(kResThreads), 0, stream, a);
    return hipGetLastError();
  }
#define KVEVICT_KEYDIFF_CASE(V)                                                              \
  case V:                                                                                    \
    if (keys.paged)                                                                          \
      hipLaunchKernelGGL((score_keydiff_kernel<V, true, false>), grid, block, 0, stream, a);  \
    else if (pair_ok)                                                                        \
      hipLaunchKernelGGL((score_keydiff_kernel<V, false, true>), grid, block, 0, stream, a);  \
    else                                                                                     \
      hipLaunchKernelGGL((score_keydiff_kernel<V, false, false>), grid, block, 0, stream, a); \
    break;
  switch (a.vpr) {
    KVEVICT_KEYDIFF_CASE(1)
    KVEVICT_KEYDIFF_CASE(2)
    KVEVICT_KEYDIFF_CASE(4)
    KVEVICT_KEYDIFF_CASE(8)
    KVEVICT_KEYDIFF_CASE(16)
    KVEVICT_KEYDIFF_CASE(32)
    KVEVICT_KEYDIFF_CASE(64)
    default:
      return hipErrorInvalidValue;  // D/8 must be a power of two <= 64
  }
#undef KVEVICT_KEYDIFF_CASE
  return hipGetLastError();
}

}  // namespace kvevict
