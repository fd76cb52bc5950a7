// Lock criterion of SURELOCK (gist.science/es/paper/2602.06412, section 2,
// "Deteccion de Convergencia"): per token, the KL divergence of its current
// posterior over the vocabulary from the previous step's,
//     D = KL(p_t || p_{t-1}),  p = softmax(logits),
// and a token that may be locked locks once D < eps; a locked token stays
// locked.  One workgroup per token row streams both logit rows once:
//     KL = sum_i p_i (x_i - y_i) - (LSE(x) - LSE(y))
//        = S / Z_x - (m_x + log Z_x) + (m_y + log Z_y)
// with Z_x = sum e^{x_i - m_x}, S = sum e^{x_i - m_x} (x_i - y_i) and Z_y
// likewise over y, kept per thread with running maxima (exponentials in
// float32 with the accurate expf, sums in float64) and reduced over the
// workgroup in a fixed order, so the result is bitwise reproducible.

#include <math.h>

#include "ba_internal.h"

namespace ba {
namespace {

constexpr int kKlThreads = 512;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct KlPart {
  float mx, my;   // running maxima (log space)
  double zx, s, zy;
};

__device__ __forceinline__ float bf16_to_f32(unsigned short u) { return __uint_as_float((unsigned)u << 16); }

// Loads 8 consecutive logits of a row as float32 (16-byte loads for bf16,
// two for float32).
template <typename T>
__device__ __forceinline__ void load8(const T* row, int64_t i, float (&o)[8]) {
  if constexpr (sizeof(T) == 2) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(row + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[2 * j] = __uint_as_float(w[j] << 16);
      o[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
  } else {
    const u32x4 a = *reinterpret_cast<const u32x4*>(row + i);
    const u32x4 b = *reinterpret_cast<const u32x4*>(row + i + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[j] = __uint_as_float(a[j]);
      o[4 + j] = __uint_as_float(b[j]);
    }
  }
}

template <typename T>
__device__ __forceinline__ float load1(const T* row, int64_t i) {
  if constexpr (sizeof(T) == 2) return bf16_to_f32(reinterpret_cast<const unsigned short*>(row)[i]);
  else return row[i];
}

// Adds elements x[0..n) / y[0..n) to the running part.
__device__ __forceinline__ void accumulate(KlPart& a, const float* x, const float* y, int n) {
  float cx = -INFINITY, cy = -INFINITY;
  for (int j = 0; j < n; ++j) {
    cx = fmaxf(cx, x[j]);
    cy = fmaxf(cy, y[j]);
  }
  if (cx > a.mx) {
    const double r = (double)expf(a.mx - cx);   // 0 when the old max is -inf
    a.zx *= r;
    a.s *= r;
    a.mx = cx;
  }
  if (cy > a.my) {
    a.zy *= (double)expf(a.my - cy);
    a.my = cy;
  }
  for (int j = 0; j < n; ++j) {
    // (a running max still at -inf means every term so far has weight 0)
    const float ex = a.mx == -INFINITY ? 0.0f : expf(x[j] - a.mx);
    a.zx += ex;
    // a zero-weight term adds nothing even where x - y is not finite
    if (ex > 0.0f) a.s += (double)ex * ((double)x[j] - (double)y[j]);
    a.zy += a.my == -INFINITY ? 0.0f : expf(y[j] - a.my);
  }
}

__device__ __forceinline__ void combine(KlPart& a, const KlPart& b) {
  const float mx = fmaxf(a.mx, b.mx), my = fmaxf(a.my, b.my);
  const double ra = a.mx == -INFINITY ? 0.0 : (double)expf(a.mx - mx);
  const double rb = b.mx == -INFINITY ? 0.0 : (double)expf(b.mx - mx);
  a.zx = a.zx * ra + b.zx * rb;
  a.s = a.s * ra + b.s * rb;
  a.mx = mx;
  const double qa = a.my == -INFINITY ? 0.0 : (double)expf(a.my - my);
  const double qb = b.my == -INFINITY ? 0.0 : (double)expf(b.my - my);
  a.zy = a.zy * qa + b.zy * qb;
  a.my = my;
}

template <typename T>
__global__ void __launch_bounds__(kKlThreads) kl_lock_kernel(const KlParams p) {
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const T* x = static_cast<const T*>(p.cur) + (int64_t)row * p.stride;
  const T* y = static_cast<const T*>(p.prev) + (int64_t)row * p.stride;
  KlPart a{-INFINITY, -INFINITY, 0.0, 0.0, 0.0};
  const int64_t V = p.vocab;
  if (p.vec) {
    // 8 logits per load, 4 loads of each row in flight per thread
    const int64_t n8 = V / 8;
    for (int64_t c0 = t; c0 < n8; c0 += 4 * kKlThreads) {
      float xs[4][8], ys[4][8];
      int cnt = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t c = c0 + (int64_t)u * kKlThreads;
        if (c < n8) {
          load8(x, c * 8, xs[u]);
          load8(y, c * 8, ys[u]);
          cnt = u + 1;
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (u < cnt) accumulate(a, xs[u], ys[u], 8);
    }
    for (int64_t i = n8 * 8 + t; i < V; i += kKlThreads) {
      const float xv = load1(x, i), yv = load1(y, i);
      accumulate(a, &xv, &yv, 1);
    }
  } else {
    for (int64_t i = t; i < V; i += kKlThreads) {
      const float xv = load1(x, i), yv = load1(y, i);
      accumulate(a, &xv, &yv, 1);
    }
  }
  // fixed-order tree over the workgroup
  __shared__ KlPart red[kKlThreads];
  red[t] = a;
  __syncthreads();
  for (int s = kKlThreads / 2; s > 0; s >>= 1) {
    if (t < s) combine(red[t], red[t + s]);
    __syncthreads();
  }
  if (t != 0) return;
  const KlPart r = red[0];
  const double lse_x = (double)r.mx + log(r.zx);
  const double lse_y = (double)r.my + log(r.zy);
  double kl = r.s / r.zx - lse_x + lse_y;
  if (kl < 0.0) kl = 0.0;   // rounding below the exact minimum of 0
  if (p.kl) p.kl[row] = (float)kl;
  if (p.locked) {
    const bool may = p.eligible ? p.eligible[row] != 0 : true;
    if (may && kl < p.eps) p.locked[row] = 1;
  }
}

}  // namespace

hipError_t launch_kl_lock(const KlParams& p, hipStream_t s) {
  if (p.n == 0) return hipSuccess;
  if (p.esize == 2)
    hipLaunchKernelGGL(kl_lock_kernel<uint16_t>, dim3(p.n), dim3(kKlThreads), 0, s, p);
  else
    hipLaunchKernelGGL(kl_lock_kernel<float>, dim3(p.n), dim3(kKlThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace ba
