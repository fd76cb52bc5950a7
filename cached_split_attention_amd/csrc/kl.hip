// Lock criterion of SURELOCK (gist.science/es/paper/2602.06412, section 2,
// "Deteccion de Convergencia"): per token, the KL divergence of its current
// posterior over the vocabulary from the previous step's,
//     D = KL(p_t || p_{t-1}),  p = softmax(logits),
// and a token that may be locked locks once D < eps; a locked token stays
// locked.  One workgroup per token row streams both logit rows once:
//     KL = sum_i p_i (x_i - y_i) - (LSE(x) - LSE(y))
//        = S / Z_x - LSE(x) + LSE(y)
// with Z_x = sum 2^(c x_i - m_x), S = sum 2^(c x_i - m_x) (x_i - y_i) and Z_y
// likewise over y, c = log2(e) rounded to float32, m a shift per thread.
//
// Numerics.  Each term is one float32 fma and one hardware exp2, so every
// term is exp((1 + e) x_i - m ln 2) with one common e = c / log2(e) - 1
// (|e| < 2^-24) and its own rounding; with LSE = m ln 2 + ln Z and S / Z
// scaled by c / log2(e) in float64, the result is the exact KL of the logits
// scaled by 1 + e, up to the rounding of the terms and sums.  The shift m is
// not a running maximum: a thread keeps its shift until a chunk's terms sum
// past 2^64 (or a term is not finite), and only then takes the chunk's
// maximum as the new shift, rescales its sums and redoes the chunk with the
// guards that -inf logits need (a zero-weight term adds nothing to S even
// where x - y is not finite).  Terms are summed per 8-element chunk in
// float32 and the chunk sums added in float64; the workgroup reduces under
// its largest shift in float64 in a fixed order, so the result is bitwise
// reproducible.

#include <float.h>
#include <math.h>

#include "ba_internal.h"

namespace ba {
namespace {

constexpr int kKlThreads = 512;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct KlPart {
  float mx, my;   // shifts (log2 units)
  double zx, s, zy;
};

__device__ __forceinline__ float bf16_to_f32(unsigned short u) { return __uint_as_float((unsigned)u << 16); }

// Loads 8 consecutive logits of a row as float32 (one 16-byte load for bf16,
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

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kChunkLimit = 0x1p64f;   // a chunk sum above this moves the shift

// Guarded step: new shifts from the chunk's maxima where they exceed the
// current ones (sums rescaled in float64), then the chunk's terms.
__device__ __forceinline__ void accumulate_guarded(KlPart& a, const float* x, const float* y, int n) {
  float cx = -INFINITY, cy = -INFINITY;
  for (int j = 0; j < n; ++j) {
    cx = fmaxf(cx, x[j]);
    cy = fmaxf(cy, y[j]);
  }
  const float nx = cx * kLog2e, ny = cy * kLog2e;
  if (nx > a.mx) {
    const double r = a.mx == -INFINITY ? 0.0 : exp2((double)a.mx - (double)nx);
    a.zx *= r;
    a.s *= r;
    a.mx = nx;
  }
  if (ny > a.my) {
    a.zy *= a.my == -INFINITY ? 0.0 : exp2((double)a.my - (double)ny);
    a.my = ny;
  }
  // a shift still at -inf (every logit so far -inf) is used as -FLT_MAX so
  // that the terms come out 0, not NaN
  const float mx = fmaxf(a.mx, -FLT_MAX), my = fmaxf(a.my, -FLT_MAX);
  float zx = 0.0f, sx = 0.0f, zy = 0.0f;
  for (int j = 0; j < n; ++j) {
    const float ex = __builtin_amdgcn_exp2f(fmaf(x[j], kLog2e, -mx));
    zx += ex;
    if (ex > 0.0f) sx = fmaf(ex, x[j] - y[j], sx);
    zy += __builtin_amdgcn_exp2f(fmaf(y[j], kLog2e, -my));
  }
  a.zx += zx;
  a.s += sx;
  a.zy += zy;
}

// Fast step under the current shifts; falls back to the guarded step when
// the chunk overflows the limit or yields a NaN (the first chunk always
// does: the shifts start at -inf).
__device__ __forceinline__ void accumulate8(KlPart& a, const float (&x)[8], const float (&y)[8]) {
  float zx = 0.0f, sx = 0.0f, zy = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float ex = __builtin_amdgcn_exp2f(fmaf(x[j], kLog2e, -a.mx));
    zx += ex;
    sx = fmaf(ex, x[j] - y[j], sx);
    zy += __builtin_amdgcn_exp2f(fmaf(y[j], kLog2e, -a.my));
  }
  if (zx <= kChunkLimit && zy <= kChunkLimit && sx == sx) {
    a.zx += zx;
    a.s += sx;
    a.zy += zy;
  } else {
    accumulate_guarded(a, x, y, 8);
  }
}

__device__ __forceinline__ double shfl_xor_f64(double v, int m) {
  const int lo = __shfl_xor(__double2loint(v), m), hi = __shfl_xor(__double2hiint(v), m);
  return __hiloint2double(hi, lo);
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
    // 8 logits per chunk, KU chunks of each row loaded before any is summed;
    // every load is issued (a chunk past the end re-reads the last one and
    // is not summed), so the loads are not split by waits.
    constexpr int KU = 4;
    const int64_t n8 = V / 8;
    for (int64_t c0 = t; c0 < n8; c0 += KU * kKlThreads) {
      float xs[KU][8], ys[KU][8];
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        const int64_t c = min(c0 + (int64_t)u * kKlThreads, n8 - 1);
        load8(x, c * 8, xs[u]);
        load8(y, c * 8, ys[u]);
      }
#pragma unroll
      for (int u = 0; u < KU; ++u)
        if (c0 + (int64_t)u * kKlThreads < n8) accumulate8(a, xs[u], ys[u]);
    }
    for (int64_t i = n8 * 8 + t; i < V; i += kKlThreads) {
      const float xv = load1(x, i), yv = load1(y, i);
      accumulate_guarded(a, &xv, &yv, 1);
    }
  } else {
    for (int64_t i = t; i < V; i += kKlThreads) {
      const float xv = load1(x, i), yv = load1(y, i);
      accumulate_guarded(a, &xv, &yv, 1);
    }
  }
  // Workgroup reduction: the largest shifts (wave shuffles, then the waves
  // in order), every thread's sums rescaled to them in float64, then summed
  // by an xor butterfly per wave (the same value in every lane) and the
  // waves' sums added in wave order.
  constexpr int kWaves = kKlThreads / 64;
  __shared__ float s_mx[kWaves], s_my[kWaves];
  __shared__ double s_sum[3][kWaves];
  const int w = t >> 6, lane = t & 63;
  float mx = a.mx, my = a.my;
  for (int m = 32; m > 0; m >>= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, m));
    my = fmaxf(my, __shfl_xor(my, m));
  }
  if (lane == 0) {
    s_mx[w] = mx;
    s_my[w] = my;
  }
  __syncthreads();
  mx = s_mx[0];
  my = s_my[0];
  for (int i = 1; i < kWaves; ++i) {
    mx = fmaxf(mx, s_mx[i]);
    my = fmaxf(my, s_my[i]);
  }
  const double r = a.mx == -INFINITY ? 0.0 : exp2((double)a.mx - (double)mx);
  const double q = a.my == -INFINITY ? 0.0 : exp2((double)a.my - (double)my);
  double zx = a.zx * r, sxy = a.s * r, zy = a.zy * q;
  for (int m = 1; m < 64; m <<= 1) {
    zx += shfl_xor_f64(zx, m);
    sxy += shfl_xor_f64(sxy, m);
    zy += shfl_xor_f64(zy, m);
  }
  if (lane == 0) {
    s_sum[0][w] = zx;
    s_sum[1][w] = sxy;
    s_sum[2][w] = zy;
  }
  __syncthreads();
  if (t != 0) return;
  zx = s_sum[0][0];
  sxy = s_sum[1][0];
  zy = s_sum[2][0];
  for (int i = 1; i < kWaves; ++i) {
    zx += s_sum[0][i];
    sxy += s_sum[1][i];
    zy += s_sum[2][i];
  }
  const double kLn2 = 0.69314718055994530942;
  const double lse_x = (double)mx * kLn2 + log(zx);
  const double lse_y = (double)my * kLn2 + log(zy);
  double kl = ((double)kLog2e / 1.44269504088896340736) * (sxy / zx) - lse_x + lse_y;
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
