// Reuse gates of FlashBlock (gist.science/es/paper/2602.05305, section 2,
// "Estrategias de Reutilizacion Adaptativa"):
//   count  - M_b = number of block positions whose Q, K or V row changed
//            (bitwise) since the previous step; reuse iff M_b < tau;
//   cosine - per head, the cosine of the block Q against the previous step's,
//            accumulated in float64; reuse iff cos > gamma.
// Both are one launch.  Workgroups publish partial results, take a ticket
// with an integer atomic, and the last workgroup of each sequence (count) or
// (sequence, head) (cosine) finishes the reduction in a fixed order and
// resets its ticket, so the workspace is zero again when the launch ends.
// Only integer atomics are used; float64 partials are summed in chunk order,
// so results are bitwise reproducible.  Partials cross workgroups (and XCDs)
// through agent-scope stores and loads, never through whole-cache flushes.

#include <math.h>

#include "ba_internal.h"

namespace ba {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ T ld_agent(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
__device__ __forceinline__ void st_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename W>
__device__ __forceinline__ bool words_differ(const W& x, const W& y) {
  if constexpr (sizeof(W) == 16) {
    return (x[0] != y[0]) | (x[1] != y[1]) | (x[2] != y[2]) | (x[3] != y[3]);
  } else {
    return x != y;
  }
}

// Does any Q, K or V row of block position (b, pos) differ between cur and
// prev?  The position's words (Q heads, then K heads, then V heads; W = the
// comparison word) are spread over the workgroup, 8 per thread per round,
// with all of a round's loads issued before any comparison so a round costs
// one memory latency.
template <typename W>
__device__ bool position_changed(const GateParams& p, int b, int pos) {
  const int wpr = p.d * p.esize / (int)sizeof(W);
  const int nq = p.hq * wpr;
  const int nk = p.k_cur ? p.hkv * wpr : 0;
  const int nv = p.v_cur ? p.hkv * wpr : 0;
  const int total = nq + nk + nv;
  constexpr int U = 8;
  bool diff = false;
  for (int t0 = threadIdx.x; t0 < total; t0 += U * (int)blockDim.x) {
    W x[U], y[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int w = t0 + u * (int)blockDim.x;
      x[u] = W{};
      y[u] = W{};
      if (w < total) {
        const void* cur = p.q_cur;
        const void* prev = p.q_prev;
        int64_t s0 = p.qs0, s1 = p.qs1, s2 = p.qs2;
        if (w >= nq) {
          w -= nq;
          const bool isv = w >= nk;
          if (isv) w -= nk;
          cur = isv ? p.v_cur : p.k_cur;
          prev = isv ? p.v_prev : p.k_prev;
          s0 = p.ks0;
          s1 = p.ks1;
          s2 = p.ks2;
        }
        const int hh = w / wpr, wi = w - hh * wpr;
        const int64_t off = ((int64_t)b * s0 + (int64_t)pos * s1 + (int64_t)hh * s2) * p.esize;
        x[u] = reinterpret_cast<const W*>(static_cast<const char*>(cur) + off)[wi];
        y[u] = reinterpret_cast<const W*>(static_cast<const char*>(prev) + off)[wi];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) diff |= words_differ(x[u], y[u]);
  }
  return diff;
}

template <typename W>
__global__ void __launch_bounds__(256) gate_count_kernel(const GateParams p) {
  const int pos = blockIdx.x, b = blockIdx.y;
  bool diff = false;
  if (p.upd_mask) {
    diff = threadIdx.x == 0 && p.upd_mask[(int64_t)b * p.n_blk + pos] != 0;
  } else {
    diff = position_changed<W>(p, b, pos);
  }
  diff = __syncthreads_or(diff);
  // One atomic per workgroup carries both the ticket (low 16 bits) and the
  // count of changed positions (high 16 bits); the last workgroup of the
  // sequence reads the total from its own return value and resets the word.
  __shared__ int s_m;
  if (threadIdx.x == 0) {
    const unsigned old = atomicAdd(reinterpret_cast<unsigned*>(p.ws_int) + b, (diff ? 0x10000u : 0u) + 1u);
    s_m = -1;
    if ((int)(old & 0xffffu) == p.n_blk - 1) {
      s_m = (int)(old >> 16) + (diff ? 1 : 0);
      atomicExch(p.ws_int + b, 0);
      p.m_count[b] = s_m;
    }
  }
  __syncthreads();
  const int m = s_m;
  if (m < 0) return;
  const uint8_t dec = (p.cache_valid && m < p.tau) ? 1 : 0;
  for (int h = threadIdx.x; h < p.hq; h += blockDim.x) p.decision[(int64_t)b * p.hq + h] = dec;
}

__device__ __forceinline__ float load_elem(const void* base, int64_t idx, int esize) {
  if (esize == 2) {
    const uint16_t u = static_cast<const uint16_t*>(base)[idx];
    return __uint_as_float((unsigned)u << 16);
  }
  return static_cast<const float*>(base)[idx];
}

__global__ void __launch_bounds__(256) gate_cos_kernel(const GateParams p) {
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int per = (p.n_blk + p.chunks - 1) / p.chunks;
  const int p0 = min(p.n_blk, c * per), p1 = min(p.n_blk, p0 + per);
  const int n = (p1 - p0) * p.d;
  double dot = 0.0, nc = 0.0, np = 0.0;
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    const int pos = p0 + e / p.d, dd = e - (e / p.d) * p.d;
    const int64_t idx = (int64_t)b * p.qs0 + (int64_t)pos * p.qs1 + (int64_t)h * p.qs2 + dd;
    const double x = load_elem(p.q_cur, idx, p.esize);
    const double y = load_elem(p.q_prev, idx, p.esize);
    dot = fma(x, y, dot);
    nc = fma(x, x, nc);
    np = fma(y, y, np);
  }
  __shared__ double red[3][256];
  red[0][threadIdx.x] = dot;
  red[1][threadIdx.x] = nc;
  red[2][threadIdx.x] = np;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) {
      red[0][threadIdx.x] += red[0][threadIdx.x + s];
      red[1][threadIdx.x] += red[1][threadIdx.x + s];
      red[2][threadIdx.x] += red[2][threadIdx.x + s];
    }
    __syncthreads();
  }
  if (threadIdx.x != 0) return;
  const int64_t bh = (int64_t)b * p.hq + h;
  double* part = p.ws_dbl + (bh * p.chunks + c) * 3;
  st_agent(part + 0, red[0][0]);
  st_agent(part + 1, red[1][0]);
  st_agent(part + 2, red[2][0]);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // partials acknowledged before the ticket
  int32_t* ticket = p.ws_int + bh;
  const int t = atomicAdd(ticket, 1);
  if (t != p.chunks - 1) return;
  // The XCD's L2 may hold stale lines of the partials: drop them first.
  asm volatile("buffer_inv sc1\n\ts_waitcnt vmcnt(0)" ::: "memory");
  double sd = 0.0, sc = 0.0, sp = 0.0;
  for (int k = 0; k < p.chunks; ++k) {
    double* q = p.ws_dbl + (bh * p.chunks + k) * 3;
    sd += ld_agent(q + 0);
    sc += ld_agent(q + 1);
    sp += ld_agent(q + 2);
    st_agent(q + 0, 0.0);
    st_agent(q + 1, 0.0);
    st_agent(q + 2, 0.0);
  }
  atomicExch(ticket, 0);
  double cs = 0.0;
  uint8_t dec = 0;
  if (sc != 0.0 && sp != 0.0) {
    cs = sd / (sqrt(sc) * sqrt(sp));
    dec = (p.cache_valid && cs > p.gamma) ? 1 : 0;
  }
  if (p.cos) p.cos[bh] = cs;
  p.decision[bh] = dec;
}

}  // namespace

int gate_cos_chunks(int n_blk, int d) {
  const int64_t elems = (int64_t)n_blk * d;
  int64_t c = (elems + 8191) / 8192;
  if (c < 1) c = 1;
  if (c > 64) c = 64;
  if (c > n_blk) c = n_blk > 0 ? n_blk : 1;
  return (int)c;
}

size_t gate_workspace_bytes(int mode, int n_seq, int hq, int n_blk, int d) {
  if (mode == BA_GATE_COUNT) return (size_t)n_seq * sizeof(int32_t);
  const size_t nbh = (size_t)n_seq * hq;
  const size_t ints = (nbh * sizeof(int32_t) + 15) & ~(size_t)15;
  return ints + nbh * gate_cos_chunks(n_blk, d) * 3 * sizeof(double);
}

hipError_t launch_gate(const GateParams& p, hipStream_t s) {
  if (p.n_seq == 0 || p.n_blk == 0) return hipSuccess;
  if (p.mode == BA_GATE_COUNT) {
    dim3 grid(p.n_blk, p.n_seq);
    if (p.vec16)
      hipLaunchKernelGGL(gate_count_kernel<u32x4>, grid, dim3(256), 0, s, p);
    else if (p.esize == 4)
      hipLaunchKernelGGL(gate_count_kernel<uint32_t>, grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(gate_count_kernel<uint16_t>, grid, dim3(256), 0, s, p);
  } else {
    dim3 grid(p.chunks, p.hq, p.n_seq);
    hipLaunchKernelGGL(gate_cos_kernel, grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace ba
