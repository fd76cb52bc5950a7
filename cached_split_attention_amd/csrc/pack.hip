// Varlen packing of unlocked query positions across branches (BlockBatch,
// gist.science/fr/paper/2605.29233, "Methodologie", "Optimisation Systeme";
// locked positions issue no query: SURELOCK, gist.science/es/paper/2602.06412,
// section 2, "Accion de Bloqueo").
// Kernel 1 (one workgroup of 16 waves): per-branch unlocked counts with wave
// ballots, an exclusive scan over branches (cu_seqlens, total), then the
// stable compaction writing gather_idx.  Kernel 2 (one workgroup per packed
// row) copies the selected Q rows into the packed buffer.  All integer,
// deterministic.

#include "ba_internal.h"

namespace ba {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct PackArgs {
  PackParams p;
  int32_t starts[kMaxBranches + 1];
};

__global__ void __launch_bounds__(1024) pack_index_kernel(const PackArgs a) {
  const PackParams& p = a.p;
  __shared__ int32_t cnt[kMaxBranches + 1];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nw = blockDim.x >> 6;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int br = wv; br < p.n_branch; br += nw) {
    const int s = a.starts[br], e = a.starts[br + 1];
    int c = 0;
    for (int base = s; base < e; base += 64) {
      const int pos = base + lane;
      const bool u = pos < e && p.locked[pos] == 0;
      c += __popcll(__ballot(u));
    }
    if (lane == 0) cnt[br] = c;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int br = 0; br < p.n_branch; ++br) {
      const int c = cnt[br];
      cnt[br] = run;
      p.cu[br] = run;
      run += c;
    }
    cnt[p.n_branch] = run;
    p.cu[p.n_branch] = run;
    *p.total = run;
  }
  __syncthreads();
  for (int br = wv; br < p.n_branch; br += nw) {
    const int s = a.starts[br], e = a.starts[br + 1];
    int run = cnt[br];
    for (int base = s; base < e; base += 64) {
      const int pos = base + lane;
      const bool u = pos < e && p.locked[pos] == 0;
      const uint64_t mask = __ballot(u);
      if (u) p.gather[run + __popcll(mask & below)] = pos;
      run += __popcll(mask);
    }
  }
  for (int r = cnt[p.n_branch] + threadIdx.x; r < p.n_total; r += blockDim.x) p.gather[r] = -1;
}

__global__ void __launch_bounds__(256) pack_copy_kernel(const PackParams p) {
  const int r = blockIdx.x;
  if (r >= *p.total) return;
  const int pos = p.gather[r];
  const int rb = p.d * p.esize;  // bytes per head row
  const char* src = static_cast<const char*>(p.q_src);
  char* dst = static_cast<char*>(p.q_packed) + (int64_t)r * p.h * rb;
  if (p.vec16) {
    const int wpr = rb / 16;
    for (int t = threadIdx.x; t < p.h * wpr; t += blockDim.x) {
      const int hh = t / wpr, wi = t - hh * wpr;
      const int64_t off = ((int64_t)pos * p.qs0 + (int64_t)hh * p.qs1) * p.esize;
      reinterpret_cast<u32x4*>(dst + (int64_t)hh * rb)[wi] = reinterpret_cast<const u32x4*>(src + off)[wi];
    }
  } else {
    const int wpr = rb / 2;
    for (int t = threadIdx.x; t < p.h * wpr; t += blockDim.x) {
      const int hh = t / wpr, wi = t - hh * wpr;
      const int64_t off = ((int64_t)pos * p.qs0 + (int64_t)hh * p.qs1) * p.esize;
      reinterpret_cast<uint16_t*>(dst + (int64_t)hh * rb)[wi] = reinterpret_cast<const uint16_t*>(src + off)[wi];
    }
  }
}

}  // namespace

hipError_t launch_pack(const PackParams& p, const int32_t* starts_host, hipStream_t s) {
  PackArgs a;
  a.p = p;
  for (int i = 0; i <= p.n_branch; ++i) a.starts[i] = starts_host[i];
  hipLaunchKernelGGL(pack_index_kernel, dim3(1), dim3(1024), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.q_src && p.n_total > 0) {
    hipLaunchKernelGGL(pack_copy_kernel, dim3(p.n_total), dim3(256), 0, s, p);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace ba
