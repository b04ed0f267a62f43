// GateSight-style weighted scores (GateSight Sec. 4.1: a fixed weight per GDN
// head over the signals of the up-to-six GDN layers preceding an attention
// layer; the log effective write log(beta*|v|)).
//
//   s[l][h][t] = sum_{slot} sum_j w[l][h][slot][j] * ln(beta[g][t][j] * vnorm[g][t][j]),
//   g = win_begin[l] + slot,   +inf for t < prot.
//
// Layout of the work: a workgroup of 256 threads owns a tile of 64 tokens.
// It walks the GDN layers g used by any window once; for each it loads the
// tile's beta and |v| rows (coalesced along the GDN heads), takes one binary64
// log per (t, j) into LDS (transposed, so lane = token reads are conflict
// free), and every wave folds that layer into the accumulators of the
// attention layers whose window contains g.  Wave w serves KV head h0 + w,
// lane = token; the weights are wave-uniform and come through scalar loads.
// Accumulation is binary64, rounded once to fp32 on the store, so the result
// matches a binary64 evaluation of the sum up to the summation order.
#include <cmath>

#include "kvevict_device.hpp"
#include "kvevict_launch.hpp"

namespace kvevict {
namespace {

constexpr int kThreads = 256;
constexpr int kTok = 64;            // tokens per tile (= lanes)
constexpr int kHeadsPerBlock = 4;   // one KV head per wave
constexpr int kLayersPerLaunch = 16;
constexpr int kJChunk = 64;         // GDN heads staged per pass
constexpr int kXStride = kTok + 1;  // doubles per staged GDN head (padding)

struct WeightedArgs {
  float* scores;
  int64_t ld;
  const float* beta;
  const float* vnorm;
  int64_t sg, st, sj;
  const float* w;
  int32_t w_slots, H, Hg, n, prot;
  int32_t l0, nl;  // attention layers [l0, l0 + nl) of this launch
  int32_t h0;      // first KV head of this launch
  int32_t g_lo, g_hi;
  WindowTable win;
};

__global__ __launch_bounds__(kThreads) void score_weighted_kernel(WeightedArgs a) {
  __shared__ double s_x[kJChunk * kXStride];
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int32_t t0 = blockIdx.x * kTok;
  const int32_t t = t0 + lane;
  const int32_t h = a.h0 + wave;
  const bool head_ok = h < a.H;

  double acc[kLayersPerLaunch];
#pragma unroll
  for (int q = 0; q < kLayersPerLaunch; ++q) acc[q] = 0.0;

  const bool tile_in_prompt = (t0 + kTok <= a.prot);
  if (!tile_in_prompt) {
    for (int32_t g = a.g_lo; g < a.g_hi; ++g) {
      for (int32_t j0 = 0; j0 < a.Hg; j0 += kJChunk) {
        const int32_t jn = min(kJChunk, a.Hg - j0);
        // stage ln(beta * |v|) of tokens [t0, t0+64) x heads [j0, j0+jn):
        // every wave first issues its 16 row loads, then takes the logs
        constexpr int kRows = kTok / kHeadsPerBlock;
        float bv[kRows], vv[kRows];
        const bool lane_ok = lane < jn;
#pragma unroll
        for (int k = 0; k < kRows; ++k) {
          const int32_t tt = t0 + wave + k * kHeadsPerBlock;
          bv[k] = 1.0f;
          vv[k] = 1.0f;
          if (lane_ok && tt < a.n) {
            const int64_t e = (int64_t)g * a.sg + (int64_t)tt * a.st + (int64_t)(j0 + lane) * a.sj;
            bv[k] = a.beta[e];
            vv[k] = a.vnorm[e];
          }
        }
        if (lane_ok) {
#pragma unroll
          for (int k = 0; k < kRows; ++k)
            s_x[lane * kXStride + wave + k * kHeadsPerBlock] = log((double)bv[k] * (double)vv[k]);
        }
        __syncthreads();
        if (head_ok) {
#pragma unroll
          for (int q = 0; q < kLayersPerLaunch; ++q) {
            if (q < a.nl) {
              const int32_t l = a.l0 + q;
              const int32_t slot = g - a.win.begin[l];
              if (slot >= 0 && slot < a.win.count[l]) {
                const float* wr = a.w + (((int64_t)l * a.H + h) * a.w_slots + slot) * a.Hg + j0;
                double s = acc[q];
                for (int32_t j = 0; j < jn; ++j) s = fma((double)wr[j], s_x[j * kXStride + lane], s);
                acc[q] = s;
              }
            }
          }
        }
        __syncthreads();
      }
    }
  }
  if (head_ok && t < a.n) {
#pragma unroll
    for (int q = 0; q < kLayersPerLaunch; ++q) {
      if (q < a.nl) {
        const int32_t l = a.l0 + q;
        a.scores[((int64_t)l * a.H + h) * a.ld + t] = (t < a.prot) ? INFINITY : (float)acc[q];
      }
    }
  }
}

}  // namespace

hipError_t launch_score_weighted(float* scores, int64_t ld, const float* beta, const float* vnorm,
                                 int64_t sg, int64_t st, int64_t sj, const float* w,
                                 int32_t w_slots, const WindowTable& win, int32_t L, int32_t H,
                                 int32_t Hg, int32_t n, int32_t prot, hipStream_t stream) {
  if (n == 0 || L == 0 || H == 0) return hipSuccess;
  const unsigned tiles = (unsigned)((n + kTok - 1) / kTok);
  for (int32_t l0 = 0; l0 < L; l0 += kLayersPerLaunch) {
    const int32_t nl = (L - l0 < kLayersPerLaunch) ? L - l0 : kLayersPerLaunch;
    int32_t g_lo = 0x7fffffff, g_hi = 0;
    for (int32_t l = l0; l < l0 + nl; ++l) {
      if (win.count[l] <= 0) continue;
      g_lo = (win.begin[l] < g_lo) ? win.begin[l] : g_lo;
      g_hi = (win.begin[l] + win.count[l] > g_hi) ? win.begin[l] + win.count[l] : g_hi;
    }
    if (g_hi <= g_lo) g_lo = g_hi = 0;  // empty windows: scores are 0 (or +inf in the prompt)
    for (int32_t h0 = 0; h0 < H; h0 += kHeadsPerBlock) {
      WeightedArgs a;
      a.scores = scores;
      a.ld = ld;
      a.beta = beta;
      a.vnorm = vnorm;
      a.sg = sg;
      a.st = st;
      a.sj = sj;
      a.w = w;
      a.w_slots = w_slots;
      a.H = H;
      a.Hg = Hg;
      a.n = n;
      a.prot = prot;
      a.l0 = l0;
      a.nl = nl;
      a.h0 = h0;
      a.g_lo = g_lo;
      a.g_hi = g_hi;
      a.win = win;
      hipLaunchKernelGGL(score_weighted_kernel, dim3(tiles), dim3(kThreads), 0, stream, a);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace kvevict
