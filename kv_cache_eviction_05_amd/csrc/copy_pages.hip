// Whole-page copy between K/V page pools through two page-id lists (GateSight
// Sec. 4.3: the cache is a pool of fixed-size blocks addressed through
// per-layer block tables, and a block can move as a unit).
//
//   K_dst page dst_ids[i] = K_src page src_ids[i]   and the same for V,  i < count.
//
// This is what the paged gather does when every slot of a destination page is
// kept in order, with the per-row index lookup taken out: the same pages
// behind the same random tables, moved as plain 16-byte vectors.  It serves as
// the copy ceiling the paged gather is measured against.  One 256-thread
// workgroup per page pair; each thread loads all its vectors of K and of V
// (nontemporal) before it stores any, like the gather.  A page id outside its
// pool skips the pair and counts it in *errors.
#include "kvevict_device.hpp"
#include "kvevict_launch.hpp"

namespace kvevict {
namespace {

constexpr int kThreads = 256;
constexpr int kPer = 8;  // vectors of K and of V per thread per step: 32 KiB per workgroup step
constexpr int64_t kMaxGrid = 1 << 23;

typedef uint32_t vec4u __attribute__((ext_vector_type(4)));

struct CopyArgs {
  const vec4u* k_src;
  const vec4u* v_src;
  vec4u* k_dst;
  vec4u* v_dst;
  const int32_t* src_ids;
  const int32_t* dst_ids;
  int64_t src_pages, dst_pages, count, page_vecs;
  uint32_t* errors;
};

__global__ __launch_bounds__(kThreads) void copy_pages_kernel(CopyArgs a) {
  for (int64_t item = blockIdx.x; item < a.count; item += gridDim.x) {
    const int32_t sp = a.src_ids[item], dp = a.dst_ids[item];
    if (sp < 0 || sp >= a.src_pages || dp < 0 || dp >= a.dst_pages) {
      if (threadIdx.x == 0 && a.errors) atomicAdd(a.errors, 1u);
      continue;
    }
    const vec4u* __restrict__ ks = a.k_src + (int64_t)sp * a.page_vecs;
    const vec4u* __restrict__ vs = a.v_src + (int64_t)sp * a.page_vecs;
    vec4u* __restrict__ kd = a.k_dst + (int64_t)dp * a.page_vecs;
    vec4u* __restrict__ vd = a.v_dst + (int64_t)dp * a.page_vecs;
    for (int64_t base = 0; base < a.page_vecs; base += kPer * kThreads) {
      vec4u x[kPer], y[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int64_t v = base + threadIdx.x + u * kThreads;
        if (v < a.page_vecs) {
          x[u] = __builtin_nontemporal_load(ks + v);
          y[u] = __builtin_nontemporal_load(vs + v);
        }
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int64_t v = base + threadIdx.x + u * kThreads;
        if (v < a.page_vecs) {
          __builtin_nontemporal_store(x[u], kd + v);
          __builtin_nontemporal_store(y[u], vd + v);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_copy_pages(const void* k_src, const void* v_src, int64_t src_pages,
                             const int32_t* src_ids, void* k_dst, void* v_dst, int64_t dst_pages,
                             const int32_t* dst_ids, int64_t count, int64_t page_bytes,
                             uint32_t* errors, hipStream_t stream) {
  if (count == 0) return hipSuccess;
  CopyArgs a;
  a.k_src = static_cast<const vec4u*>(k_src);
  a.v_src = static_cast<const vec4u*>(v_src);
  a.k_dst = static_cast<vec4u*>(k_dst);
  a.v_dst = static_cast<vec4u*>(v_dst);
  a.src_ids = src_ids;
  a.dst_ids = dst_ids;
  a.src_pages = src_pages;
  a.dst_pages = dst_pages;
  a.count = count;
  a.page_vecs = page_bytes / 16;
  a.errors = errors;
  const int64_t grid = count < kMaxGrid ? count : kMaxGrid;
  hipLaunchKernelGGL(copy_pages_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvevict
