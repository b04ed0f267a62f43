// GateSight-style weighted scores (GateSight Sec. 4.1: a fixed weight per GDN
// head over the signals of the up-to-six GDN layers preceding an attention
// layer; the log effective write log(beta*|v|)).
//
//   s[l][h][t] = sum_{slot} sum_j w[l][h][slot][j] * ln(beta[g][t][j] * vnorm[g][t][j]),
//   g = win_begin[l] + slot,   +inf for t < prot.
//
// Layout of the work.  A workgroup of eight waves owns a tile of 64 tokens
// and walks the GDN layers g of its launch once, in order, in passes of 48
// GDN heads.  For each (g, pass) the workgroup loads the tile of beta and |v|
// with coalesced 8-byte loads (when the layout allows) and the pass's weights
// of the active windows; every thread takes the binary64 logs of the six
// products it loaded into a transposed LDS tile, and the weights go to LDS as
// binary64.  The next tile's loads are issued before the current one is
// folded.  Wave w then owns GDN heads [6w, 6w + 6) with lane = token: it folds
// its six logs into partial sums, one per (KV head, accumulator slot).  A slot
// holds the attention layer whose window contains g; the host assigns slots
// so that layers with overlapping windows never share one (at most kSlots at
// a time, else more launches) and passes, per GDN layer, each slot's weight
// row and the windows that end there.  When a layer's window ends, each wave
// leaves its partial sums in LDS; right after the next step's barrier the
// first four waves add them in wave order and store the fp32 score while the
// other waves fold (no barriers of its own).  The LDS tiles are double-
// buffered, so each step needs one barrier.
//
// Each thread's offsets within a full tile are computed once; a step adds only
// the GDN layer and pass offsets.  The log table holds {ln c, 1/c} pairs, so a
// log makes one 16-byte LDS read.
//
// Signals in the usual layout (48 heads per 16-byte aligned token row, unit
// head stride) take a second kernel with the same arithmetic in the same
// order, whose tiles go from HBM straight into LDS (see
// score_weighted_lds_kernel below); other layouts take this one.
//
// Precision: the product beta*|v| of two floats is exact in binary64; its
// natural log is taken in binary64 (table-driven reduction to [-2^-9, 2^-9]
// and a degree-6 series, within a few binary64 ulps; zero, infinities, NaN
// and negative products go through the library log); accumulation is
// binary64 and the result is rounded once to fp32.
#include <cmath>
#include <type_traits>

#include "kvevict_device.hpp"
#include "kvevict_launch.hpp"

namespace kvevict {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kTok = 64;                    // tokens per tile (= lanes)
static_assert(kThreads == kWeightedThreads && kTok == kWeightedTile, "the grid checks");
constexpr int kJW = 6;                      // GDN heads per wave per pass
constexpr int kJPass = kWaves * kJW;        // GDN heads per pass
constexpr int kHB = 4;                      // KV heads per launch
constexpr int kSlots = 2;                   // accumulator slots
constexpr int kLayersPerLaunch = 16;
constexpr int kPlanLayers = 64;             // GDN layers one launch spans
constexpr int kLnTable = 256;               // ln table: centres of [1, 2) in steps of 1/256
constexpr int kXStride = kTok + 1;          // doubles per staged GDN head (padding)
constexpr int kElems = kTok * kJPass / kThreads;  // tile elements per thread
constexpr int kWRow = kSlots * kHB * kJPass;      // weights of one (GDN layer, pass)
static_assert(kTok * kJPass == kElems * kThreads, "the tile splits evenly over the threads");
static_assert(kWRow <= kThreads, "one weight per thread");

struct WeightedArgs {
  int64_t ld;
  int64_t sg, st, sj;
  int32_t w_slots, H, Hg, n, prot;
  int32_t h0, hb;   // KV heads [h0, h0 + hb) of this launch
  int32_t nl;       // attention layers of this launch
  int32_t g_lo, g_hi;
  uint32_t empty_mask;                   // launch layers with an empty window
  int32_t layer[kLayersPerLaunch];       // attention layer of each launch layer
  int32_t slot[kLayersPerLaunch];        // its accumulator slot
  int64_t woff[kPlanLayers][kSlots];     // weight row of (g, slot) for head h0, or -1
  uint32_t end_mask[kPlanLayers];        // launch layers whose window ends at g
  uint32_t* hist0;                       // first-level bins of a global top-B, or null
};

constexpr int kFirstLevelBins = kGlobalFirstLevelBins;  // rank key bits [21, 32)
constexpr int kFirstLevelShift = 21;

// ln(x) in binary64 for a positive normal x: x = 2^e * m, m in [1, 2);
// c = 1 + (i + 1/2)/256 is the centre of m's slot, r = m/c - 1 (one fma with
// the tabulated 1/c: absolute error ~2^-53) with |r| <= 2^-9, and
// ln x = e ln 2 + ln c + ln(1 + r) with ln(1 + r) = r - r^2/2 + ... - r^6/6
// (truncation below 2^-66).  Only the high word of x carries e and i.  *special is set when x is not a positive
// normal number (zero, subnormal, infinite, NaN or negative).
__device__ __forceinline__ double ln_fast(double x, const double2* tab, bool* special) {
  const uint32_t hi = (uint32_t)__double2hiint(x);
  const uint32_t ex = hi >> 20;  // sign and biased exponent
  *special = ex - 1u >= 0x7feu;
  const uint32_t i = (hi >> 12) & (kLnTable - 1);
  const double m = __hiloint2double((int)((hi & 0x000fffffu) | 0x3ff00000u), __double2loint(x));
  const double2 tc = tab[i];  // {ln c, 1/c}
  const double r = fma(m, tc.y, -1.0);
  double p = -1.0 / 6.0;
  p = fma(p, r, 1.0 / 5.0);
  p = fma(p, r, -0.25);
  p = fma(p, r, 1.0 / 3.0);
  p = fma(p, r, -0.5);
  p = fma(p, r, 1.0);
  return fma((double)((int32_t)ex - 1023), M_LN2, fma(p, r, tc.x));
}

// The library log, out of line, for the arguments ln_fast does not take.
__device__ __attribute__((noinline)) double ln_special(double x) { return log(x); }

// A thread's share of one (GDN layer, pass) tile: tokens [t0, t0 + 64) x GDN
// heads [j0, j0 + jn), element e = token * jn + j; the thread holds the VW
// consecutive heads of vectors q = tid + k * kThreads.
template <int VW>
struct Tile {
  static constexpr int kVecs = kElems / VW;
  float b[kVecs][VW];
  float v[kVecs][VW];
  float w;  // one weight of the (GDN layer, pass): [slot][head][j]
};

// Element position of vector k in a tile of width jn (kFull: jn == kJPass).
template <int VW, bool kFull>
__device__ __forceinline__ void tile_pos(int k, int32_t jn, int32_t* tok, int32_t* j) {
  const int32_t q = threadIdx.x + k * kThreads;
  const int32_t vpt = (kFull ? kJPass : jn) / VW;  // vectors per token
  *tok = q / vpt;
  *j = (q - *tok * vpt) * VW;
}

// Loads a tile and this thread's weight (1.0 signals outside the data, so
// their log is 0; weight 0 outside the active rows).  VW = 2 needs sj == 1,
// even jn and 8-byte aligned rows.
template <int VW, bool kFull>
__device__ __forceinline__ void load_tile(const WeightedArgs& a, const float* __restrict__ beta,
                                          const float* __restrict__ vnorm,
                                          const float* __restrict__ wts, int32_t g, int32_t p,
                                          int32_t t0, Tile<VW>& r, const int64_t* off) {
  const int32_t j0 = p * kJPass;
  const int32_t jn = kFull ? kJPass : min(kJPass, a.Hg - j0);
  const int64_t base = (int64_t)g * a.sg + (int64_t)j0 * a.sj;
#pragma unroll
  for (int k = 0; k < Tile<VW>::kVecs; ++k) {
#pragma unroll
    for (int c = 0; c < VW; ++c) {
      r.b[k][c] = 1.0f;
      r.v[k][c] = 1.0f;
    }
    int64_t e;
    if (kFull) {
      if (off[k] < 0) continue;
      e = base + off[k];
    } else {
      int32_t tok, j;
      tile_pos<VW, kFull>(k, jn, &tok, &j);
      if (tok >= kTok || t0 + tok >= a.n) continue;
      e = base + (int64_t)(t0 + tok) * a.st + (int64_t)j * a.sj;
    }
    if (VW == 2) {
      const float2 x = *reinterpret_cast<const float2*>(beta + e);
      const float2 y = *reinterpret_cast<const float2*>(vnorm + e);
      r.b[k][0] = x.x;
      r.b[k][VW - 1] = x.y;
      r.v[k][0] = y.x;
      r.v[k][VW - 1] = y.y;
    } else {
      r.b[k][0] = beta[e];
      r.v[k][0] = vnorm[e];
    }
  }
  r.w = 0.0f;
  if (threadIdx.x < kWRow) {
    const int32_t s = threadIdx.x / (kHB * kJPass);
    const int32_t hh = (threadIdx.x / kJPass) % kHB;
    const int32_t j = threadIdx.x % kJPass;
    const int64_t wo = a.woff[g - a.g_lo][s];
    if (wo >= 0 && hh < a.hb && j < jn)
      r.w = wts[wo + (int64_t)hh * a.w_slots * a.Hg + j0 + j];
  }
}

// Logs of a loaded tile into x[j][token] (transposed) and its weights, as
// binary64, into w.
template <int VW, bool kFull>
__device__ __forceinline__ void stage_tile(const Tile<VW>& r, int32_t jn, double* x, double* w,
                                           const double2* tab) {
  double y[Tile<VW>::kVecs][VW];
  bool any_special = false;
#pragma unroll
  for (int k = 0; k < Tile<VW>::kVecs; ++k)
#pragma unroll
    for (int c = 0; c < VW; ++c) {
      bool sp;
      y[k][c] = ln_fast((double)r.b[k][c] * (double)r.v[k][c], tab, &sp);
      any_special |= sp;
    }
  if (any_special) {  // zero, infinite, NaN or negative signals: the library log
#pragma unroll
    for (int k = 0; k < Tile<VW>::kVecs; ++k)
#pragma unroll
      for (int c = 0; c < VW; ++c) {
        const double xv = (double)r.b[k][c] * (double)r.v[k][c];
        const uint32_t ex = (uint32_t)__double2hiint(xv) >> 20;
        if (ex - 1u >= 0x7feu) y[k][c] = ln_special(xv);
      }
  }
#pragma unroll
  for (int k = 0; k < Tile<VW>::kVecs; ++k) {
    int32_t tok, j;
    tile_pos<VW, kFull>(k, jn, &tok, &j);
    if (!kFull && tok >= kTok) continue;
#pragma unroll
    for (int c = 0; c < VW; ++c) x[(j + c) * kXStride + tok] = y[k][c];
  }
  if (threadIdx.x < kWRow) w[threadIdx.x] = (double)r.w;
}

// Adds the scores this workgroup stored (every layer and head of the launch,
// tokens [t0, t0 + kTok) from prot on) to the first-level bins of a global
// top-B: an LDS histogram of their rank keys' top 11 bits, then one
// device-scope add per nonzero bin.  The caller has passed a barrier after the
// stores, so they are visible to the whole workgroup.
__device__ void add_first_level_bins(const WeightedArgs& a, const float* scores, int32_t t0,
                                     uint32_t* s_h) {
  const int tid = threadIdx.x;
  for (int b = tid; b < kFirstLevelBins; b += kThreads) s_h[b] = 0u;
  __syncthreads();
  const int32_t total = a.nl * a.hb * kTok;
  for (int32_t e = tid; e < total; e += kThreads) {
    const int32_t tt = t0 + e % kTok;
    const int32_t rest = e / kTok;
    const int32_t hh = rest % a.hb, q = rest / a.hb;
    if (tt >= a.prot && tt < a.n) {
      const float v = scores[((int64_t)a.layer[q] * a.H + a.h0 + hh) * a.ld + tt];
      atomicAdd(&s_h[rank_key(v) >> kFirstLevelShift], 1u);
    }
  }
  __syncthreads();
  for (int b = tid; b < kFirstLevelBins; b += kThreads) {
    const uint32_t h = s_h[b];
    if (h) __hip_atomic_fetch_add(a.hist0 + b, h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The weights, signals and scores come as separate restrict-qualified
// arguments: the kernel never writes what it reads.
template <int VW>
__global__ __launch_bounds__(kThreads) void score_weighted_kernel(WeightedArgs a,
                                                                  const float* __restrict__ wts,
                                                                  const float* __restrict__ beta,
                                                                  const float* __restrict__ vnorm,
                                                                  float* __restrict__ scores) {
  __shared__ double2 s_tab[kLnTable];
  __shared__ double s_x[2][kJPass * kXStride];
  __shared__ double s_w[2][kWRow];
  __shared__ double s_red[kWaves][kHB][kTok];
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int32_t t0 = blockIdx.x * kTok;
  const int32_t t = t0 + lane;

  // stores the fp32 score of (layer index q of the launch, head h0 + hh) for the tile
  auto store = [&](int q, int hh, int32_t tt, double v) {
    if (hh < a.hb && tt < a.n)
      scores[((int64_t)a.layer[q] * a.H + a.h0 + hh) * a.ld + tt] =
          (tt < a.prot) ? INFINITY : (float)v;
  };
  // layers with an empty window score 0; a tile inside the prompt is all +inf
  const bool tile_in_prompt = (t0 + kTok <= a.prot);
  if (wave < kHB) {
    for (int q = 0; q < a.nl; ++q)
      if (tile_in_prompt || ((a.empty_mask >> q) & 1u)) store(q, wave, t, 0.0);
  }
  if (tile_in_prompt) return;
  if (a.g_hi > a.g_lo) {  // some window of the launch is not empty
    if (tid < kLnTable) {
      const double c = 1.0 + ((double)tid + 0.5) * (1.0 / kLnTable);
      s_tab[tid] = make_double2(log(c), 1.0 / c);
    }

    const int32_t passes = (a.Hg + kJPass - 1) / kJPass;
    const bool full = a.Hg % kJPass == 0;  // every pass is kJPass heads wide
    const int32_t steps = (a.g_hi - a.g_lo) * passes;
    double acc[kHB][kSlots];
#pragma unroll
    for (int hh = 0; hh < kHB; ++hh)
#pragma unroll
      for (int s = 0; s < kSlots; ++s) acc[hh][s] = 0.0;

    // offsets of this thread's vectors within a full tile (-1 past the last token)
    int64_t off[Tile<VW>::kVecs];
#pragma unroll
    for (int k = 0; k < Tile<VW>::kVecs; ++k) {
      int32_t tok, j;
      tile_pos<VW, true>(k, kJPass, &tok, &j);
      off[k] = (t0 + tok < a.n) ? (int64_t)(t0 + tok) * a.st + (int64_t)j * a.sj : -1;
    }
    Tile<VW> regs;
    if (full)
      load_tile<VW, true>(a, beta, vnorm, wts, a.g_lo, 0, t0, regs, off);
    else
      load_tile<VW, false>(a, beta, vnorm, wts, a.g_lo, 0, t0, regs, off);
    __syncthreads();  // the ln table
    // A window that ends leaves each wave's partial sums in s_red; they are
    // added (in wave order) and stored right after the next step's barrier, by
    // the first kHB waves, while the others go on folding.  s_red is written
    // again only at the next window end; when that comes at the very next
    // step, a barrier first lets the pending sums be read.
    int32_t pending = -1;       // launch layer whose sums wait in s_red
    int32_t pending_step = -2;  // the step whose barrier they are added after
    auto reduce_store = [&](int32_t q) {
      if (tid < kHB * kTok) {
        const int hh = tid / kTok;
        double v = 0.0;
#pragma unroll
        for (int w2 = 0; w2 < kWaves; ++w2) v += s_red[w2][hh][lane];
        store(q, hh, t, v);
      }
    };
    for (int32_t step = 0; step < steps; ++step) {
      const int32_t g = a.g_lo + step / passes;
      const int32_t p = step - (g - a.g_lo) * passes;
      const int32_t jn = min(kJPass, a.Hg - p * kJPass);
      double* x = s_x[step & 1];
      double* w = s_w[step & 1];
      if (full)
        stage_tile<VW, true>(regs, jn, x, w, s_tab);
      else
        stage_tile<VW, false>(regs, jn, x, w, s_tab);
      if (step + 1 < steps) {  // the next tile streams in while this one is folded
        const int32_t g2 = a.g_lo + (step + 1) / passes;
        const int32_t p2 = step + 1 - (g2 - a.g_lo) * passes;
        if (full)
          load_tile<VW, true>(a, beta, vnorm, wts, g2, p2, t0, regs, off);
        else
          load_tile<VW, false>(a, beta, vnorm, wts, g2, p2, t0, regs, off);
      }
      __syncthreads();
      if (pending >= 0) {
        reduce_store(pending);
        pending = -1;
        pending_step = step;
      }

      const int32_t jb = wave * kJW;  // this wave's heads [jb, je) of the tile
      const int32_t je = min(jb + kJW, jn);
      const int32_t gi = g - a.g_lo;
      // folds logs [jb, je) into the partial sums; kFull: je - jb == kJW
      auto fold = [&](auto full_tag) {
        constexpr bool kFull = decltype(full_tag)::value;
        double xv[kJW];
#pragma unroll
        for (int k = 0; k < kJW; ++k)
          xv[k] = (kFull || jb + k < je) ? x[(jb + k) * kXStride + lane] : 0.0;
#pragma unroll
        for (int s = 0; s < kSlots; ++s) {
          if (a.woff[gi][s] < 0) continue;
#pragma unroll
          for (int hh = 0; hh < kHB; ++hh) {
            const double* wr = w + (s * kHB + hh) * kJPass + jb;
            double v = acc[hh][s];
#pragma unroll
            for (int k = 0; k < kJW; ++k)
              if (kFull || jb + k < je) v = fma(wr[k], xv[k], v);
            acc[hh][s] = v;
          }
        }
      };
      if (je - jb == kJW)
        fold(std::true_type{});
      else if (jb < je)
        fold(std::false_type{});

      if (p + 1 < passes) continue;
      // windows ending at g: add the waves' partial sums in a fixed order and store
      uint32_t ends = a.end_mask[gi];
      while (ends) {
        const int32_t q = __builtin_ctz(ends);
        ends &= ends - 1u;
        const int32_t s_q = a.slot[q];
        if (pending >= 0) {  // a second window ends at this step: add the first one now
          __syncthreads();
          reduce_store(pending);
          pending = -1;
          pending_step = step;
        }
        if (pending_step == step) __syncthreads();  // s_red was read after this step's barrier
#pragma unroll
        for (int s = 0; s < kSlots; ++s) {
          if (s == s_q) {
#pragma unroll
            for (int hh = 0; hh < kHB; ++hh) {
              s_red[wave][hh][lane] = acc[hh][s];
              acc[hh][s] = 0.0;
            }
          }
        }
        pending = q;
      }
    }
    if (pending >= 0) {
      __syncthreads();
      reduce_store(pending);
    }
  }
  if (a.hist0) {
    __syncthreads();  // the tile's scores are stored and the LDS tiles are free
    add_first_level_bins(a, scores, t0, reinterpret_cast<uint32_t*>(&s_x[0][0]));
  }
}

// The same scores for signals laid out with 48 GDN heads per token row, 16-byte
// aligned rows and unit head stride (the usual [G, n, 48] layout): one pass
// per GDN layer, and the tiles travel from HBM straight into LDS
// (global_load_lds_dwordx4), so no register holds a tile in flight and the
// next layer's tile is requested right after a step's barrier, streaming in
// while the whole step (logs and fold) runs.  A stage holds the tile of beta
// and of |v| as 16-byte chunks of four heads, each token row padded to 13
// chunks so that 64 lanes reading one chunk of 64 consecutive tokens hit
// distinct LDS banks; each wave takes the logs of its own six heads straight
// from the stage (no transposed copy), in the same order as above, so both
// kernels give identical bits.  The two stages are separate LDS arrays and the
// step loop is unrolled by two, so that the compiler sees that reads of one
// stage do not depend on the loads in flight into the other.
constexpr int kQuads = kJPass / 4;                    // chunks of four heads per token row
constexpr int kRowChunks = kQuads + 1;                // + one pad chunk per row
constexpr int kStageChunks = kTok * kRowChunks;       // 832 chunks per signal per stage
constexpr int kSigLoads = kStageChunks / kWave;       // 13 wave loads per signal per stage
constexpr int kSigWaves = kWaves / 2;                 // waves loading one signal
constexpr int kLoadsPerWave = (kSigLoads + kSigWaves - 1) / kSigWaves;
static_assert(kStageChunks % kWave == 0, "a stage is whole wave loads");
static_assert(kJPass % 4 == 0 && kJW % 2 == 0, "heads in whole chunks, pairs per wave");
static_assert(kWRow % (kJPass * kHB) == 0 && (kJPass * kHB) % kWave == 0,
              "a weight slot is whole waves");
static_assert(kSlots == 2, "the window-end branch names both slots");
static_assert(kFirstLevelBins * 4 <= kStageChunks * 16, "the bins fit a stage");

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// A workgroup barrier that orders LDS accesses only: it does not wait for the
// tile loads in flight, as a full barrier (with its memory fence) would.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__global__ __launch_bounds__(kThreads) void score_weighted_lds_kernel(
    WeightedArgs a, const float* __restrict__ wts, const float* __restrict__ beta,
    const float* __restrict__ vnorm, float* __restrict__ scores) {
  __shared__ v4f s_b0[kStageChunks], s_v0[kStageChunks];  // stage 0: beta, |v|
  __shared__ v4f s_b1[kStageChunks], s_v1[kStageChunks];  // stage 1
  __shared__ double s_w0[kWRow], s_w1[kWRow];
  __shared__ double2 s_tab[kLnTable];
  __shared__ double s_red[kWaves][kHB][kTok];
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int32_t t0 = blockIdx.x * kTok;
  const int32_t t = t0 + lane;

  auto store = [&](int q, int hh, int32_t tt, double v) {
    if (hh < a.hb && tt < a.n)
      scores[((int64_t)a.layer[q] * a.H + a.h0 + hh) * a.ld + tt] =
          (tt < a.prot) ? INFINITY : (float)v;
  };
  const bool tile_in_prompt = (t0 + kTok <= a.prot);
  if (wave < kHB) {
    for (int q = 0; q < a.nl; ++q)
      if (tile_in_prompt || ((a.empty_mask >> q) & 1u)) store(q, wave, t, 0.0);
  }
  if (tile_in_prompt) return;
  if (a.g_hi > a.g_lo) {
    if (tid < kLnTable) {
      const double c = 1.0 + ((double)tid + 0.5) * (1.0 / kLnTable);
      s_tab[tid] = make_double2(log(c), 1.0 / c);
    }
    const int32_t steps = a.g_hi - a.g_lo;
    double acc[kHB][kSlots];
#pragma unroll
    for (int hh = 0; hh < kHB; ++hh)
#pragma unroll
      for (int s = 0; s < kSlots; ++s) acc[hh][s] = 0.0;

    // Waves [0, 4) load beta, [4, 8) |v|: wave load i of a signal fills stage chunks
    // [64 i, 64 i + 64), chunk c = token * 13 + quad.  This lane's offsets within a GDN
    // layer (-1: a pad chunk or a token past n, not loaded; its stale slot only feeds
    // that token, whose scores are not stored).
    const int sw = wave % kSigWaves;
    const bool loads_v = wave >= kSigWaves;
    int64_t off[kLoadsPerWave];
#pragma unroll
    for (int k = 0; k < kLoadsPerWave; ++k) {
      const int i = sw + k * kSigWaves;
      const int32_t c = i * kWave + lane;
      const int32_t tok = c / kRowChunks, q = c % kRowChunks;
      off[k] = (i < kSigLoads && q < kQuads && t0 + tok < a.n)
                   ? (int64_t)(t0 + tok) * a.st + 4 * q : -1;
    }
    auto issue_into = [&](v4f* stage_sig, const float* sig, int32_t g) __attribute__((always_inline)) {
      const float* src = sig + (int64_t)g * a.sg;
#pragma unroll
      for (int k = 0; k < kLoadsPerWave; ++k) {
        const int i = sw + k * kSigWaves;
        if (i >= kSigLoads) break;
        if (off[k] >= 0)
          __builtin_amdgcn_global_load_lds(src + off[k], (lds_void*)(stage_sig + i * kWave), 16,
                                           0, 0);
      }
    };
    auto issue = [&](auto stage, int32_t g) __attribute__((always_inline)) {
      if constexpr (decltype(stage)::value == 0) {
        if (loads_v) issue_into(s_v0, vnorm, g);
        else issue_into(s_b0, beta, g);
      } else {
        if (loads_v) issue_into(s_v1, vnorm, g);
        else issue_into(s_b1, beta, g);
      }
    };
    // one weight of the (GDN layer) per thread of waves [0, 6): slot wave / 3
    const int32_t w_slot = wave / (kHB * kJPass / kWave);
    auto load_w = [&](int32_t g) {
      float w = 0.0f;
      if (w_slot < kSlots) {
        const int32_t hh = (tid / kJPass) % kHB;
        const int32_t j = tid % kJPass;
        const int64_t wo = a.woff[g - a.g_lo][w_slot];
        if (wo >= 0 && hh < a.hb) w = wts[wo + (int64_t)hh * a.w_slots * a.Hg + j];
      }
      return w;
    };
    issue(std::integral_constant<int, 0>{}, a.g_lo);
    float wnext = load_w(a.g_lo);
    if (tid < kWRow) s_w0[tid] = (double)wnext;

    int32_t pending = -1, pending_step = -2;
    // the waves' partial sums of a finished window, added in wave order; read in one
    // block that waits for its own reads (the tile loads in flight go elsewhere)
    auto reduce_store = [&](int32_t q) __attribute__((always_inline)) {
      if (tid < kHB * kTok) {
        const int hh = tid / kTok;
        const uint32_t ar = (uint32_t)reinterpret_cast<uintptr_t>(&s_red[0][hh][lane]);
        double r0, r1, r2, r3, r4, r5, r6, r7;
        static_assert(kWaves == 8 && kHB * kTok * 8 == 2048, "offsets below");
        asm volatile(
            "ds_read_b64 %0, %8\n\t"
            "ds_read_b64 %1, %8 offset:2048\n\t"
            "ds_read_b64 %2, %8 offset:4096\n\t"
            "ds_read_b64 %3, %8 offset:6144\n\t"
            "ds_read_b64 %4, %8 offset:8192\n\t"
            "ds_read_b64 %5, %8 offset:10240\n\t"
            "ds_read_b64 %6, %8 offset:12288\n\t"
            "ds_read_b64 %7, %8 offset:14336\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6),
              "=&v"(r7)
            : "v"(ar)
            : "memory");
        double v = 0.0;
        v += r0;
        v += r1;
        v += r2;
        v += r3;
        v += r4;
        v += r5;
        v += r6;
        v += r7;
        store(q, hh, t, v);
      }
    };
    const int32_t jb = wave * kJW;  // this wave's heads [jb, jb + 6)
    auto body = [&](auto stage, int32_t step) __attribute__((always_inline)) {
      constexpr int kCur = decltype(stage)::value;
      const v4f* sb = kCur == 0 ? s_b0 : s_b1;
      const v4f* sv = kCur == 0 ? s_v0 : s_v1;
      const double* w = kCur == 0 ? s_w0 : s_w1;
      double* w_next = kCur == 0 ? s_w1 : s_w0;
      const int32_t g = a.g_lo + step;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's part of the stage
      __syncthreads();  // the whole stage is in LDS, and the other one was read
      if (step + 1 < steps) {  // the next layer streams in during this step
        wnext = load_w(g + 1);
        issue(std::integral_constant<int, 1 - kCur>{}, g + 1);
      }
      if (pending >= 0) {
        reduce_store(pending);
        pending = -1;
        pending_step = step;
      }
      // this wave's six heads for token `lane`, read in one block that waits for its own
      // reads (the compiler cannot tell these addresses from the loads in flight)
      const uint32_t ab = (uint32_t)reinterpret_cast<uintptr_t>(sb + lane * kRowChunks) + jb * 4;
      const uint32_t av = (uint32_t)reinterpret_cast<uintptr_t>(sv + lane * kRowChunks) + jb * 4;
      uint64_t rb0, rb1, rb2, rv0, rv1, rv2;
      asm volatile(
          "ds_read_b64 %0, %6\n\t"
          "ds_read_b64 %1, %6 offset:8\n\t"
          "ds_read_b64 %2, %6 offset:16\n\t"
          "ds_read_b64 %3, %7\n\t"
          "ds_read_b64 %4, %7 offset:8\n\t"
          "ds_read_b64 %5, %7 offset:16\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(rb0), "=&v"(rb1), "=&v"(rb2), "=&v"(rv0), "=&v"(rv1), "=&v"(rv2)
          : "v"(ab), "v"(av)
          : "memory");
      const uint64_t rb[3] = {rb0, rb1, rb2}, rv[3] = {rv0, rv1, rv2};
      float bv[kJW], vv[kJW];
#pragma unroll
      for (int k = 0; k < kJW / 2; ++k) {
        bv[2 * k] = __uint_as_float((uint32_t)rb[k]);
        bv[2 * k + 1] = __uint_as_float((uint32_t)(rb[k] >> 32));
        vv[2 * k] = __uint_as_float((uint32_t)rv[k]);
        vv[2 * k + 1] = __uint_as_float((uint32_t)(rv[k] >> 32));
      }
      double xv[kJW];
      bool any_special = false;
#pragma unroll
      for (int k = 0; k < kJW; ++k) {
        bool sp;
        xv[k] = ln_fast((double)bv[k] * (double)vv[k], s_tab, &sp);
        any_special |= sp;
      }
      if (any_special) {
#pragma unroll
        for (int k = 0; k < kJW; ++k) {
          const double xp = (double)bv[k] * (double)vv[k];
          const uint32_t ex = (uint32_t)__double2hiint(xp) >> 20;
          if (ex - 1u >= 0x7feu) xv[k] = ln_special(xp);
        }
      }
      const int32_t gi = g - a.g_lo;
#pragma unroll
      for (int s = 0; s < kSlots; ++s) {
        if (a.woff[gi][s] < 0) continue;
#pragma unroll
        for (int hh = 0; hh < kHB; ++hh) {
          const double* wr = w + (s * kHB + hh) * kJPass + jb;
          double v = acc[hh][s];
#pragma unroll
          for (int k = 0; k < kJW; ++k) v = fma(wr[k], xv[k], v);
          acc[hh][s] = v;
        }
      }
      // the next layer's weights (that row was last read in step - 1)
      if (step + 1 < steps && tid < kWRow) w_next[tid] = (double)wnext;

      uint32_t ends = a.end_mask[gi];
      while (ends) {
        const int32_t q = __builtin_ctz(ends);
        ends &= ends - 1u;
        const int32_t s_q = a.slot[q];
        if (pending >= 0) {
          lds_barrier();
          reduce_store(pending);
          pending = -1;
          pending_step = step;
        }
        if (pending_step == step) lds_barrier();
        // selects of values (no branch per slot), so that acc stays in registers
        const bool first = s_q == 0;
#pragma unroll
        for (int hh = 0; hh < kHB; ++hh) {
          const double x0 = acc[hh][0], x1 = acc[hh][1];
          s_red[wave][hh][lane] = first ? x0 : x1;
          acc[hh][0] = first ? 0.0 : x0;
          acc[hh][1] = first ? x1 : 0.0;
        }
        pending = q;
      }
    };
    for (int32_t step = 0; step < steps; step += 2) {
      body(std::integral_constant<int, 0>{}, step);
      if (step + 1 < steps) body(std::integral_constant<int, 1>{}, step + 1);
    }
    if (pending >= 0) {
      __syncthreads();
      reduce_store(pending);
    }
  }
  if (a.hist0) {
    __syncthreads();
    add_first_level_bins(a, scores, t0, reinterpret_cast<uint32_t*>(&s_b0[0]));
  }
}

static_assert(kThreads >= kHB * kTok, "one thread per (head, token) in the reduction");
static_assert(kFirstLevelBins * 4 <= 2 * kJPass * kXStride * 8, "the bins fit the LDS tiles");
static_assert(kWaves >= kHB, "one wave per head for the direct stores");

}  // namespace

hipError_t launch_score_weighted(float* scores, int64_t ld, const float* beta, const float* vnorm,
                                 int64_t sg, int64_t st, int64_t sj, const float* w,
                                 int32_t w_slots, const WindowTable& win, int32_t L, int32_t H,
                                 int32_t Hg, int32_t n, int32_t prot, hipStream_t stream,
                                 uint32_t* hist0) {
  if (n == 0 || L == 0 || H == 0) return hipSuccess;
  if ((n + kTok - 1) / kTok > max_workgroups(kThreads)) return hipErrorInvalidConfiguration;
  const unsigned tiles = (unsigned)((n + kTok - 1) / kTok);
  const bool vec = sj == 1 && sg % 2 == 0 && st % 2 == 0 && Hg % 2 == 0 &&
                   (reinterpret_cast<uintptr_t>(beta) & 7u) == 0 &&
                   (reinterpret_cast<uintptr_t>(vnorm) & 7u) == 0;
  const bool lds_path = Hg == kJPass && sj == 1 && st % 4 == 0 && sg % 4 == 0 &&
                        (reinterpret_cast<uintptr_t>(beta) & 15u) == 0 &&
                        (reinterpret_cast<uintptr_t>(vnorm) & 15u) == 0;
  // Greedy grouping of layers into launches: a layer joins the current launch
  // in the first slot whose layers' windows it does not overlap; when no slot
  // is free, the launch is full or its GDN range would pass kPlanLayers, a
  // new launch starts.
  int32_t l = 0;
  while (l < L) {
    WeightedArgs a;
    a.ld = ld;
    a.sg = sg;
    a.st = st;
    a.sj = sj;
    a.w_slots = w_slots;
    a.H = H;
    a.Hg = Hg;
    a.n = n;
    a.prot = prot;
    a.nl = 0;
    a.empty_mask = 0u;
    a.hist0 = hist0;
    int32_t lo = 0x7fffffff, hi = 0;
    int32_t begin[kLayersPerLaunch], end[kLayersPerLaunch];
    for (; l < L && a.nl < kLayersPerLaunch; ++l) {
      const int32_t b = win.begin[l], e = win.begin[l] + win.count[l];
      int32_t slot = 0;
      if (e > b) {
        const int32_t nlo = b < lo ? b : lo, nhi = e > hi ? e : hi;
        if (nhi - nlo > kPlanLayers) break;
        for (slot = 0; slot < kSlots; ++slot) {
          bool free = true;
          for (int32_t q = 0; q < a.nl; ++q)
            if (a.slot[q] == slot && begin[q] < end[q] && begin[q] < e && b < end[q]) free = false;
          if (free) break;
        }
        if (slot == kSlots) break;  // overlaps kSlots windows of this launch: next launch
        lo = nlo;
        hi = nhi;
      } else {
        a.empty_mask |= 1u << a.nl;
      }
      a.layer[a.nl] = l;
      a.slot[a.nl] = slot;
      begin[a.nl] = b;
      end[a.nl] = e;
      ++a.nl;
    }
    if (hi <= lo) lo = hi = 0;  // only empty windows
    a.g_lo = lo;
    a.g_hi = hi;
    for (int32_t h0 = 0; h0 < H; h0 += kHB) {
      a.h0 = h0;
      a.hb = (H - h0 < kHB) ? H - h0 : kHB;
      for (int32_t gi = 0; gi < kPlanLayers; ++gi) {
        a.end_mask[gi] = 0u;
        for (int s = 0; s < kSlots; ++s) a.woff[gi][s] = -1;
      }
      for (int32_t q = 0; q < a.nl; ++q) {
        if (begin[q] >= end[q]) continue;
        for (int32_t g = begin[q]; g < end[q]; ++g)
          a.woff[g - lo][a.slot[q]] =
              (((int64_t)a.layer[q] * H + h0) * w_slots + (g - begin[q])) * Hg;
        a.end_mask[end[q] - 1 - lo] |= 1u << q;
      }
      if (lds_path)
        hipLaunchKernelGGL(score_weighted_lds_kernel, dim3(tiles), dim3(kThreads), 0, stream, a,
                           w, beta, vnorm, scores);
      else if (vec)
        hipLaunchKernelGGL(score_weighted_kernel<2>, dim3(tiles), dim3(kThreads), 0, stream, a, w,
                           beta, vnorm, scores);
      else
        hipLaunchKernelGGL(score_weighted_kernel<1>, dim3(tiles), dim3(kThreads), 0, stream, a, w,
                           beta, vnorm, scores);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace kvevict
