// Random Attention scores ("Random Attention" blog summary, Algorithm 1: a
// random score per entry, the prompt pinned to +inf).
//
// One thread evaluates one Philox4x64-10 block and writes the four slots it
// covers (slot i uses word i%4 of the block at counter i/4), as one 16-byte
// store when the row is aligned.  A block of 256 threads covers 1024 slots of
// one list; blockIdx.y walks the lists of this launch.
#include <cmath>

#include "kvevict_device.hpp"
#include "kvevict_launch.hpp"

namespace kvevict {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void score_random_kernel(
    float* __restrict__ scores, int64_t ld, int64_t list0, int32_t L, int32_t H, int32_t n,
    int32_t prot, uint64_t seed, uint32_t round, int32_t shared_draw) {
  const int64_t list = list0 + blockIdx.y;
  const int32_t c = blockIdx.x * kThreads + threadIdx.x;  // Philox block index
  const int32_t i0 = 4 * c;
  if (i0 >= n) return;

  uint64_t request, layer, head;
  if (shared_draw) {
    request = (uint64_t)(list / L);
    layer = (uint64_t)(list % L);
    head = 0;
  } else {
    const int64_t lh = (int64_t)L * H;
    request = (uint64_t)(list / lh);
    layer = (uint64_t)((list / H) % L);
    head = (uint64_t)(list % H);
  }

  float v[4];
  if (i0 + 3 < prot) {
    v[0] = v[1] = v[2] = v[3] = INFINITY;
  } else {
    const Philox4x64 r = philox4x64_10((uint64_t)c, head, layer, (request << 32) | round, seed, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = (i0 + q < prot) ? INFINITY : unit_from_word(r.w[q]);
  }

  float* row = scores + list * ld;
  if (i0 + 3 < n && ((reinterpret_cast<uintptr_t>(row + i0) & 15u) == 0)) {
    *reinterpret_cast<float4*>(row + i0) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (i0 + q < n) row[i0 + q] = v[q];
  }
}

}  // namespace

hipError_t launch_score_random(float* scores, int64_t ld, int64_t num_lists, int32_t L, int32_t H,
                               int32_t n, int32_t prot, uint64_t seed, uint32_t round,
                               bool shared_draw, hipStream_t stream) {
  if (num_lists == 0 || n == 0) return hipSuccess;
  const int32_t blocks = (n + 4 * kThreads - 1) / (4 * kThreads);
  const int64_t kMaxY = 65535;
  for (int64_t list0 = 0; list0 < num_lists; list0 += kMaxY) {
    const int64_t rows = (num_lists - list0 < kMaxY) ? num_lists - list0 : kMaxY;
    dim3 grid((unsigned)blocks, (unsigned)rows);
    hipLaunchKernelGGL(score_random_kernel, grid, dim3(kThreads), 0, stream, scores, ld, list0, L,
                       H, n, prot, seed, round, shared_draw ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kvevict
