// Standalone log-space merge of two partial attention results (FlashBlock,
// gist.science/es/paper/2602.05305, section 2, "Mecanismo Central", merge
// equation).  One group of d/4 threads per row, four float32 lanes each; the
// merged log-normaliser is m + log(e^{L1-m} + e^{L2-m}).

#include <math.h>

#include "ba_internal.h"

namespace ba {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr float kLog2e = 1.44269504088896340736f;

__global__ void __launch_bounds__(256) merge_kernel(const MergeParams p) {
  const int tpr = p.d / 4;
  const int rpb = 256 / tpr;
  const int64_t row = (int64_t)blockIdx.x * rpb + threadIdx.x / tpr;
  const int t = threadIdx.x % tpr;
  // Threads past the last row (or past rpb * tpr) only join the barrier.
  const bool valid = threadIdx.x < rpb * tpr && row < p.rows;
  float l1 = -INFINITY, l2 = -INFINITY;
  f32x4 x1 = {0.0f, 0.0f, 0.0f, 0.0f}, x2 = x1;
  if (valid) {
    l1 = p.l1[row];
    l2 = p.l2[row];
    x1 = *reinterpret_cast<const f32x4*>(p.a1 + row * p.d + 4 * t);
    x2 = *reinterpret_cast<const f32x4*>(p.a2 + row * p.d + 4 * t);
  }
  // Every read of the workgroup's rows completes before any write: a row's
  // d/4 threads can span two waves (d/4 need not divide 64), and in-place
  // use (a == a1 or a2, l == l1 or l2) must not let one wave's store of L
  // reach another wave's load of it.
  __syncthreads();
  if (!valid) return;
  const float m = fmaxf(l1, l2);
  float w1 = 0.0f, w2 = 0.0f, rden = 0.0f, lf = -INFINITY;
  if (m != -INFINITY) {
    w1 = __builtin_amdgcn_exp2f((l1 - m) * kLog2e);
    w2 = __builtin_amdgcn_exp2f((l2 - m) * kLog2e);
    const float den = w1 + w2;
    rden = 1.0f / den;
    lf = m + __logf(den);
  }
  const f32x4 y = (w1 * rden) * x1 + (w2 * rden) * x2;
  *reinterpret_cast<f32x4*>(p.a + row * p.d + 4 * t) = y;
  if (p.l && t == 0) p.l[row] = lf;
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, hipStream_t s) {
  const int rpb = 256 / (p.d / 4);
  const int64_t blocks = (p.rows + rpb - 1) / rpb;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace ba
