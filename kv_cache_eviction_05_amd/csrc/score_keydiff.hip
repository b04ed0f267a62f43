// KeyDiff key scores (GateSight Sec. 5.1 baselines paragraph: the cosine
// similarity of each key, as stored in the cache, to the unnormalised mean key
// of its head; the least similar keys are kept under flat per-head budgets).
//
//   score[list][i] = -cos(k_i, mean_j k_j)   (mean over all n keys of the list),
//   +inf for i < prot; a zero norm gives cos = 0; zero is written as +0.
//
// One workgroup of 256 threads per list, two passes over the list's keys.
// A row of D bf16 is VPR = D/8 16-byte vectors; thread t owns vector column
// t % VPR of rows t / VPR + k * (256 / VPR).  Pass 1 accumulates the column
// sums in binary64 (exact for bf16 inputs of moderate range, and in a fixed
// order), reduces them through LDS into the mean and its squared norm.  Pass 2
// re-reads the keys (largely from the caches), forms each row's dot product
// with the mean and its squared norm in binary64, adds the VPR partials of a
// row with lane shuffles, and rounds -dot/(|k||mean|) once to fp32.
#include <cmath>

#include "kvevict_device.hpp"
#include "kvevict_launch.hpp"

namespace kvevict {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

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
__device__ __forceinline__ int64_t key_row(const KeydiffArgs& a, int64_t list, int32_t t,
                                           int32_t vpr) {
  if (!a.keys.paged) return list * a.keys.list_stride_v + (int64_t)t * vpr;
  const int64_t g = list / a.H;
  const int32_t h = (int32_t)(list - g * a.H);
  const int32_t page = a.keys.page_table[g * a.keys.pt_ld + (t >> a.keys.page_shift)];
  if (page < 0 || (int64_t)page >= a.keys.capacity) return -1;
  const int64_t slot = ((int64_t)page << a.keys.page_shift) + (t & ((1 << a.keys.page_shift) - 1));
  return (slot * a.H + h) * vpr;
}

__device__ __forceinline__ vec4u load_key(const KeydiffArgs& a, int64_t list, int32_t t,
                                          int32_t vpr, int32_t col) {
  const int64_t off = key_row(a, list, t, vpr);
  return off >= 0 ? a.k[off + col] : vec4u{0u, 0u, 0u, 0u};
}

// The eight bf16 of a 16-byte vector as binary64 (exact).
__device__ __forceinline__ void unpack8(vec4u v, double* x) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    x[2 * q] = (double)__uint_as_float(v[q] << 16);
    x[2 * q + 1] = (double)__uint_as_float(v[q] & 0xffff0000u);
  }
}

template <int VPR>
__global__ __launch_bounds__(kThreads) void score_keydiff_kernel(KeydiffArgs a) {
  __shared__ double s_part[kThreads * 8];  // pass-1 partial column sums
  __shared__ double s_mean[kThreads * 8];  // the mean key, D <= 2048 entries
  __shared__ double s_red[kThreads / kWave];
  const int32_t vpr = VPR ? VPR : a.vpr;
  const int32_t D = vpr * 8;
  const int32_t rpi = kThreads / vpr;  // rows per iteration
  const int tid = threadIdx.x;
  const bool active = tid < rpi * vpr;
  const int32_t col = tid % vpr, r0 = tid / vpr;
  const int64_t list = blockIdx.x;
  const int32_t n = a.n;
  float* out = a.scores + list * a.ld;
  if (a.prot >= n) {  // every slot protected
    for (int32_t i = tid; i < n; i += kThreads) out[i] = INFINITY;
    return;
  }

  // --- pass 1: column sums ---------------------------------------------------
  double sum[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sum[e] = 0.0;
  if (active) {
    for (int32_t base = r0; base < n; base += rpi * kUnroll) {
      vec4u v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int32_t t = base + u * rpi;
        v[u] = (t < n) ? load_key(a, list, t, vpr, col) : vec4u{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        double x[8];
        unpack8(v[u], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) sum[e] += x[e];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) s_part[r0 * D + col * 8 + e] = sum[e];
  }
  __syncthreads();
  double mm_part = 0.0;
  for (int32_t d = tid; d < D; d += kThreads) {
    double s = 0.0;
    for (int32_t r = 0; r < rpi; ++r) s += s_part[r * D + d];  // fixed order
    const double mean = s / (double)n;
    s_mean[d] = mean;
    mm_part += mean * mean;
  }
  // |mean|^2: wave sums, then the waves in order
  for (int off = kWave / 2; off > 0; off >>= 1) mm_part += __shfl_xor(mm_part, off, kWave);
  if (lane_id() == 0) s_red[tid / kWave] = mm_part;
  __syncthreads();
  double mm = 0.0;
#pragma unroll
  for (int w = 0; w < kThreads / kWave; ++w) mm += s_red[w];
  const double mnorm = sqrt(mm);
  double mu[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mu[e] = active ? s_mean[col * 8 + e] : 0.0;

  // --- pass 2: per-row dot with the mean and squared norm ----------------------
  for (int32_t b0 = 0; b0 < n; b0 += rpi * kUnroll) {
    vec4u v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int32_t t = b0 + r0 + u * rpi;
      v[u] = (active && t < n) ? load_key(a, list, t, vpr, col) : vec4u{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      double x[8];
      unpack8(v[u], x);
      double dot = 0.0, kk = 0.0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        dot = fma(x[e], mu[e], dot);
        kk = fma(x[e], x[e], kk);
      }
      // add the VPR partials of the row (consecutive lanes, VPR a power of two <= 64)
      for (int off = vpr / 2; off > 0; off >>= 1) {
        dot += __shfl_xor(dot, off, kWave);
        kk += __shfl_xor(kk, off, kWave);
      }
      const int32_t t = b0 + r0 + u * rpi;
      if (active && col == 0 && t < n) {
        float sc = INFINITY;
        if (t >= a.prot) {
          const double den = sqrt(kk) * mnorm;
          sc = (den > 0.0) ? (float)(-(dot / den)) : 0.0f;
          if (sc == 0.0f) sc = 0.0f;  // -0 written as +0
        }
        out[t] = sc;
      }
    }
  }
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
  switch (a.vpr) {
    case 16:
      hipLaunchKernelGGL(score_keydiff_kernel<16>, grid, block, 0, stream, a);
      break;
    case 32:
      hipLaunchKernelGGL(score_keydiff_kernel<32>, grid, block, 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL(score_keydiff_kernel<0>, grid, block, 0, stream, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace kvevict
