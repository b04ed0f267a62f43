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
// such rows stay in registers and the next 9 (D <= 128), 8 or 7 in LDS, which
// at D = 128 holds 608 of 1088 rows between the two passes.  The other rows
// are read a second time soon after the first, and those reads mostly hit the
// Infinity Cache: measured on the 36,864-list batch, a plain read of every row
// once and of the streamed rows again takes 1.22x the time of one read;
// twelve register rows gained nothing, and one 1024-thread workgroup per CU
// holding 1024 rows (1.04x the bytes) was 14% slower, since two workgroups per
// CU let one list's reads overlap the other's arithmetic.
// Pass 1 accumulates the column sums in binary64 in a fixed order (lanes of a
// column with shuffles, then the waves in a tree through LDS) into the mean
// and its squared norm.  Pass 2 forms each row's dot product with the mean and
// its squared norm in binary64 and adds the VPR partials of a row with DPP lane
// moves; the binary64 work bounds the kernel as much as the reads do, so the
// lanes of a group collect VPR rows' sums before the square root and division,
// which then run once per row (not once per lane group), and the result
// -dot / (sqrt(|k|^2) * sqrt(|mean|^2)) is rounded once to fp32, with IEEE
// binary64 square roots and division.  The sums run in another order than a
// plain loop's, so the binary64 cosine may differ from it by a few units of
// 2^-53 times (D + n * |sum of |k_i|| / |sum of k_i|); the fp32 score then
// equals the plain loop's rounding except where that cosine lies within this
// bound of a midpoint between two fp32 values, where it may be the other
// neighbour (one fp32 ulp away).
#include <cmath>

#include "kvevict_device.hpp"
#include "kvevict_launch.hpp"

namespace kvevict {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kReg = 10;    // rows per thread held in registers
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

template <int VPR, bool kPaged>
__global__ __launch_bounds__(kThreads) void score_keydiff_kernel(KeydiffArgs a) {
  constexpr int32_t rpi = kThreads / VPR;  // rows per iteration
  constexpr int32_t D = VPR * 8;
  constexpr int kLds = lds_rows<VPR>();
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
  // streamed tail: whole steps of kUnroll rows per thread without bounds checks, then
  // the last partial step checked (the same rows in the same order either way)
  int32_t b0 = kCap;
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

}  // namespace

hipError_t launch_score_keydiff(float* scores, int64_t ld, const StoreView& keys, const void* k,
                                int32_t D, int32_t H, int64_t num_lists, int32_t n, int32_t prot,
                                hipStream_t stream) {
  if (num_lists == 0 || n == 0) return hipSuccess;
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
#define KVEVICT_KEYDIFF_CASE(V)                                                       \
  case V:                                                                             \
    if (keys.paged)                                                                   \
      hipLaunchKernelGGL((score_keydiff_kernel<V, true>), grid, block, 0, stream, a);  \
    else                                                                              \
      hipLaunchKernelGGL((score_keydiff_kernel<V, false>), grid, block, 0, stream, a); \
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
