// float32 attention on the vector ALUs (head dim 64 or 128): prefix attention
// without key splitting, and in-block attention with the fused log-space
// merge (FlashBlock, gist.science/es/paper/2602.05305, section 2, "Mecanismo
// Central").  One wave per (query row, head); keys are processed 64 at a time,
// one key per lane for the scores, one output dim per lane for P.V.  Meant
// for small float32 problems, where launch latency dominates.

#include <math.h>

#include "ba_internal.h"

namespace ba {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int D>
__global__ void __launch_bounds__(256) attn_f32_kernel(const AttnParams p) {
  constexpr int DPL = D / 64;  // output dims per lane
  __shared__ float sp[4][64];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + wv;
  const int64_t n_items = (int64_t)p.n_seq * p.max_q * p.hq;
  if (item >= n_items) return;
  const int h = (int)(item % p.hq);
  const int64_t vrow = item / p.hq;
  const int b = (int)(vrow / p.max_q);
  const int i = (int)(vrow - (int64_t)b * p.max_q);
  const bool qvar = p.cu_q != nullptr && p.q_rows == nullptr;   // packed Q rows
  const bool kvar = p.cu_k != nullptr;
  int qbase = 0, nq = p.max_q, kbase = 0, nk = p.max_k;
  if (p.cu_q) {
    qbase = p.cu_q[b];
    nq = min(max(p.cu_q[b + 1] - qbase, 0), p.max_q);
  }
  if (kvar) {
    kbase = p.cu_k[b];
    nk = p.cu_k[b + 1] - kbase;
  }
  if (i >= nq) return;
  const int qi = p.q_rows ? listed_row(p, b, qbase + i) : i;   // dense position
  if (p.mode != kBlock && p.decision && p.decision[b * p.hq + h]) return;
  const int kvh = h / p.group;

  const float* qrow = static_cast<const float*>(p.q) +
      (qvar ? (int64_t)(qbase + i) * p.qs1 : (int64_t)b * p.qs0 + (int64_t)qi * p.qs1) +
      (int64_t)h * p.qs2;
  const float* kptr = static_cast<const float*>(p.k) +
      (kvar ? (int64_t)kbase * p.ks1 : (int64_t)b * p.ks0) + (int64_t)kvh * p.ks2;
  const float* vptr = static_cast<const float*>(p.v) +
      (kvar ? (int64_t)kbase * p.vs1 : (int64_t)b * p.vs0) + (int64_t)kvh * p.vs2;

  float q[D];
#pragma unroll
  for (int c = 0; c < D; c += 4) {
    const float4 x = *reinterpret_cast<const float4*>(qrow + c);
    q[c] = x.x;
    q[c + 1] = x.y;
    q[c + 2] = x.z;
    q[c + 3] = x.w;
  }
  float o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;
  const float c2 = p.scale_log2;

  for (int t0 = 0; t0 < nk; t0 += 64) {
    const int j = t0 + lane;
    float sc = -INFINITY;
    if (j < nk) {
      const float* kr = kptr + (int64_t)j * p.ks1;
      float acc = 0.0f;
#pragma unroll
      for (int c = 0; c < D; c += 4) {
        const float4 x = *reinterpret_cast<const float4*>(kr + c);
        acc = fmaf(q[c], x.x, acc);
        acc = fmaf(q[c + 1], x.y, acc);
        acc = fmaf(q[c + 2], x.z, acc);
        acc = fmaf(q[c + 3], x.w, acc);
      }
      sc = acc * c2;
    }
    const float m_new = fmaxf(m_run, wave_max(sc));
    const float alpha = exp2f(m_run - m_new);
    const float pj = exp2f(sc - m_new);
    l_run = l_run * alpha + wave_sum(pj);
    m_run = m_new;
    sp[wv][lane] = pj;
    __builtin_amdgcn_wave_barrier();
    const int nj = min(64, nk - t0);
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] *= alpha;
    for (int jj = 0; jj < nj; ++jj) {
      const float w = sp[wv][jj];
      const float* vr = vptr + (int64_t)(t0 + jj) * p.vs1;
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] = fmaf(w, vr[lane + 64 * e], o[e]);
    }
    __builtin_amdgcn_wave_barrier();
  }

  const bool has = l_run > 0.0f;
  const float inv = has ? 1.0f / l_run : 0.0f;
  const float L = has ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
  const int64_t orow = qvar ? (int64_t)(qbase + i) : (int64_t)b * p.max_q + qi;
  const int64_t oe = orow * p.hq + h;

  if (p.mode == kPrefixFinal) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) p.a[oe * D + lane + 64 * e] = o[e] * inv;
    if (lane == 0) p.l[oe] = L;
    return;
  }
  // block mode
  if (p.a) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) p.a[oe * D + lane + 64 * e] = o[e] * inv;
  }
  if (p.l && lane == 0) p.l[oe] = L;
  if (p.a_cache) {
    const float lc = p.l_cache[oe];
    const float mm = fmaxf(lc, L);
    float wc = 0.0f, wi = 0.0f, lf = -INFINITY, rden = 0.0f;
    if (mm != -INFINITY) {
      wc = exp2f((lc - mm) * kLog2e);
      wi = exp2f((L - mm) * kLog2e);
      const float den = wc + wi;
      rden = 1.0f / den;
      lf = mm + logf(den);
    }
    if (p.a_full) {
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const int c = lane + 64 * e;
        p.a_full[oe * D + c] = (wc * rden) * p.a_cache[oe * D + c] + (wi * rden) * (o[e] * inv);
      }
    }
    if (p.l_full && lane == 0) p.l_full[oe] = lf;
  }
}

}  // namespace

hipError_t launch_attn_f32(const AttnParams& p, int d, hipStream_t s) {
  const int64_t items = (int64_t)p.n_seq * p.max_q * p.hq;
  const int64_t blocks = (items + 3) / 4;
  if (blocks == 0) return hipSuccess;
  if (d == 128)
    hipLaunchKernelGGL(attn_f32_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(attn_f32_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace ba
