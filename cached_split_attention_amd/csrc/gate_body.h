// Workgroup bodies of the two reuse gates of FlashBlock
// (gist.science/es/paper/2602.05305, section 2, "Estrategias de Reutilizacion
// Adaptativa"), shared by the stand-alone gate kernels and by the attention
// launch that runs the gate in its first workgroups:
//   count  - M_b = number of block positions whose Q, K or V row changed
//            (bitwise) since the previous step; reuse iff M_b < tau;
//   cosine - per head, the cosine of the block Q against the previous step's,
//            accumulated in float64; reuse iff cos > gamma;
//   cumulative count - as count, over the positions updated at any step since
//            the sequence's cache was last written (a per-position mark kept
//            by the caller between steps, cleared when the sequence
//            recomputes);
//   rows   - per position: is its Q row unchanged (the partial refresh
//            recomputes only the rows that changed).
// Workgroups publish partial results, take a ticket with an integer atomic,
// and the last workgroup of each sequence (count) or (sequence, head)
// (cosine) finishes the reduction in a fixed order and resets its ticket, so
// the workspace is zero again when the launch ends.  Only integer atomics
// are used; float64 partials are summed in chunk order, so results are
// bitwise reproducible for a given workgroup size.  Partials and decisions
// cross workgroups (and XCDs) through agent-scope stores and loads, never
// through whole-cache flushes.
//
// With p.ready set, the gate also publishes its result to consumers in the
// same launch through ready words (zero before the launch), kept in
// kReadyCopies copies p.ready_stride ints apart so that the many polling
// workgroups spread over several memory channels (a workgroup polls copy
// blockIdx % kReadyCopies):
//   count  - the workgroup that finishes sequence b stores kCountReady | M_b
//            in every copy of ready[b] (consumers derive the decision, the
//            same for every head, from M_b, so they need not read the
//            decision bytes);
//   cosine - the workgroup that finishes (b, h) adds 1 to every copy once
//            decision[b, h] is written, so ready[b] == hq means all of b's
//            are there.
#pragma once

#include <math.h>

#include "ba_internal.h"

namespace ba {
namespace gate {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCountReady = 1 << 30;   // count mode: ready[b] = kCountReady | M_b


template <typename T>
__device__ __forceinline__ T ld_agent(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T>
__device__ __forceinline__ void st_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Stores of this thread acknowledged (performed at the agent's coherence
// point) before whatever follows.
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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
// comparison word) are spread over the workgroup, 16 per thread per round,
// with all of a round's loads issued before any comparison so a round costs
// one memory latency.
template <typename W>
__device__ bool position_changed(const GateParams& p, int b, int pos) {
  const int wpr = p.d * p.esize / (int)sizeof(W);
  const int nq = p.hq * wpr;
  const int nk = p.k_cur ? p.hkv * wpr : 0;
  const int nv = p.v_cur ? p.hkv * wpr : 0;
  const int total = nq + nk + nv;
  constexpr int U = 16;
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

// Which of the block positions pos0 .. pos0+npos-1 of sequence b have a Q, K
// or V row that differs between cur and prev?  Returns this thread's share
// as a bit mask (bit i: position pos0+i).  The positions' words (per
// position: Q heads, then K heads, then V heads; W = the comparison word) are
// spread over the workgroup, U per thread per round, with all of a round's
// loads issued before any comparison, so a round costs one memory latency
// (one round covers 64 KB of cur and of prev at 256 threads and 16-byte
// words).
template <typename W>
__device__ unsigned positions_changed(const GateParams& p, int b, int pos0, int npos) {
  const int wpr = p.d * p.esize / (int)sizeof(W);
  const int nq = p.hq * wpr;
  const int nk = p.k_cur ? p.hkv * wpr : 0;
  const int nv = p.v_cur ? p.hkv * wpr : 0;
  const int per_pos = nq + nk + nv;
  const int total = npos * per_pos;
  constexpr int U = 16;
  unsigned mask = 0;
  for (int t0 = threadIdx.x; t0 < total; t0 += U * (int)blockDim.x) {
    W x[U], y[U];
    int pi[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int w = t0 + u * (int)blockDim.x;
      x[u] = W{};
      y[u] = W{};
      pi[u] = 0;
      if (w < total) {
        const int i = w / per_pos;
        w -= i * per_pos;
        pi[u] = i;
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
        const int64_t off = ((int64_t)b * s0 + (int64_t)(pos0 + i) * s1 + (int64_t)hh * s2) * p.esize;
        x[u] = reinterpret_cast<const W*>(static_cast<const char*>(cur) + off)[wi];
        y[u] = reinterpret_cast<const W*>(static_cast<const char*>(prev) + off)[wi];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (words_differ(x[u], y[u])) mask |= 1u << pi[u];
  }
  return mask;
}

// Count gate (and its cumulative and per-row forms), one workgroup per
// p.pos_per_wg consecutive block positions of one sequence (workgroup wg:
// sequence wg / n, group wg % n, n groups per sequence).  lds: two unsigned
// and one int of scratch.
template <typename W, bool MULTI>
__device__ void count_body(const GateParams& p, int wg, void* lds) {
  const int ppw = MULTI ? p.pos_per_wg : 1;
  const int nw = MULTI ? (p.n_blk + ppw - 1) / ppw : p.n_blk;
  const int b = wg / nw, grp = wg - b * nw;
  const int pos0 = grp * ppw, npos = MULTI ? min(ppw, p.n_blk - pos0) : 1;
  unsigned* s_mask = static_cast<unsigned*>(lds);   // [0]: changed, [1]: counted
  int* s_m = reinterpret_cast<int*>(s_mask + 2);
  // Per position: the mark (cumulative mode) or the row decision (rows
  // mode), stored and acknowledged before the ticket below, so that a clear
  // by the finishing workgroup lands after it; returns whether it counts.
  auto settle = [&](int i, bool d) {
    const int64_t pe = (int64_t)b * p.n_blk + pos0 + i;
    if (p.mode == BA_GATE_COUNT_CUM) {
      // marked if updated at any step since the last refresh (with no
      // valid cache there is none: old marks do not count)
      d = d || (p.cache_valid && ld_agent(p.since + pe) != 0);
      st_agent(p.since + pe, (uint8_t)(d ? 1 : 0));
      stores_done();
    } else if (p.mode == BA_GATE_ROWS) {
      st_agent(p.decision + pe, (uint8_t)(p.cache_valid && !d ? 1 : 0));
    }
    return d;
  };
  int c = 0;   // positions of this workgroup that count (thread 0)
  if (!MULTI || npos == 1) {
    // one position: a single word scan and a workgroup OR through the
    // scratch (not __syncthreads_or, which brings LDS of its own)
    if (threadIdx.x == 0) s_mask[0] = 0u;
    __syncthreads();
    bool diff = false;
    if (p.upd_mask) diff = threadIdx.x == 0 && p.upd_mask[(int64_t)b * p.n_blk + pos0] != 0;
    else diff = position_changed<W>(p, b, pos0);
    if (diff) s_mask[0] = 1u;
    __syncthreads();
    if (threadIdx.x == 0) c = settle(0, s_mask[0] != 0u) ? 1 : 0;
  } else {
    if (threadIdx.x < 2) s_mask[threadIdx.x] = 0u;
    __syncthreads();
    unsigned mine = 0;
    if (p.upd_mask) {
      if ((int)threadIdx.x < npos && p.upd_mask[(int64_t)b * p.n_blk + pos0 + threadIdx.x] != 0)
        mine = 1u << threadIdx.x;
    } else {
      mine = positions_changed<W>(p, b, pos0, npos);
    }
    if (mine) atomicOr(s_mask, mine);
    __syncthreads();
    // (threads i < npos <= 32 are all in the first wave)
    const int i = threadIdx.x;
    if (i < npos && settle(i, (s_mask[0] >> i) & 1u)) atomicOr(s_mask + 1, 1u << i);
    __syncthreads();
    if (threadIdx.x == 0) c = __popc(s_mask[1]);
  }
  // One atomic per workgroup carries both the ticket (low 16 bits) and the
  // count of counted positions (high 16 bits); the last workgroup of the
  // sequence reads the total from its own return value and resets the word.
  if (threadIdx.x == 0) {
    const unsigned old = atomicAdd(reinterpret_cast<unsigned*>(p.ws_int) + b, ((unsigned)c << 16) + 1u);
    *s_m = -1;
    if ((int)(old & 0xffffu) == nw - 1) {
      const int m = (int)(old >> 16) + c;
      *s_m = m;
      if (p.ready)
        for (int k = 0; k < kReadyCopies; ++k) atomicExch(p.ready + k * p.ready_stride + b, kCountReady | m);
      atomicExch(p.ws_int + b, 0);
      p.m_count[b] = m;
    }
  }
  __syncthreads();
  const int m = *s_m;
  if (m < 0 || p.mode == BA_GATE_ROWS) return;
  const uint8_t dec = (p.cache_valid && m < p.tau) ? 1 : 0;
  for (int h = threadIdx.x; h < p.hq; h += blockDim.x) st_agent(p.decision + (int64_t)b * p.hq + h, dec);
  // the cache of b is rewritten this step: nothing is updated since then
  if (p.mode == BA_GATE_COUNT_CUM && !dec)
    for (int q = threadIdx.x; q < p.n_blk; q += blockDim.x) st_agent(p.since + (int64_t)b * p.n_blk + q, (uint8_t)0);
}

__device__ __forceinline__ float load_elem(const void* base, int64_t idx, int esize) {
  if (esize == 2) {
    const uint16_t u = static_cast<const uint16_t*>(base)[idx];
    return __uint_as_float((unsigned)u << 16);
  }
  return static_cast<const float*>(base)[idx];
}

// Cosine gate, one workgroup per (position chunk c, head h, sequence b).
// red: 3 * blockDim.x doubles of LDS (blockDim.x a power of two).
__device__ void cos_body(const GateParams& p, int c, int h, int b, double* red) {
  const int nt = (int)blockDim.x, t = (int)threadIdx.x;
  const int per = (p.n_blk + p.chunks - 1) / p.chunks;
  const int p0 = min(p.n_blk, c * per), p1 = min(p.n_blk, p0 + per);
  double dot = 0.0, nc = 0.0, np = 0.0;
  if (p.vec16) {
    // 16-byte words (8 bf16 or 4 float32 of one row), U per thread issued
    // together before any is summed; each thread sums its words in order
    constexpr int U = 4;
    const int ve = 16 / p.esize, wpr = p.d / ve;
    const int n = (p1 - p0) * wpr;
    for (int w0 = t; w0 < n; w0 += U * nt) {
      u32x4 xw[U], yw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int w = w0 + u * nt;
        xw[u] = yw[u] = u32x4{0, 0, 0, 0};
        if (w < n) {
          const int pos = p0 + w / wpr, cw = w - (w / wpr) * wpr;
          const int64_t idx = (int64_t)b * p.qs0 + (int64_t)pos * p.qs1 + (int64_t)h * p.qs2 + (int64_t)cw * ve;
          xw[u] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(p.q_cur) + idx * p.esize);
          yw[u] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(p.q_prev) + idx * p.esize);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (w0 + u * nt >= n) break;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (p.esize == 2) {
            const double x0 = __uint_as_float(xw[u][j] << 16), x1 = __uint_as_float(xw[u][j] & 0xffff0000u);
            const double y0 = __uint_as_float(yw[u][j] << 16), y1 = __uint_as_float(yw[u][j] & 0xffff0000u);
            dot = fma(x0, y0, dot);
            nc = fma(x0, x0, nc);
            np = fma(y0, y0, np);
            dot = fma(x1, y1, dot);
            nc = fma(x1, x1, nc);
            np = fma(y1, y1, np);
          } else {
            const double x0 = __uint_as_float(xw[u][j]), y0 = __uint_as_float(yw[u][j]);
            dot = fma(x0, y0, dot);
            nc = fma(x0, x0, nc);
            np = fma(y0, y0, np);
          }
        }
      }
    }
  } else {
    const int n = (p1 - p0) * p.d;
    for (int e = t; e < n; e += nt) {
      const int pos = p0 + e / p.d, dd = e - (e / p.d) * p.d;
      const int64_t idx = (int64_t)b * p.qs0 + (int64_t)pos * p.qs1 + (int64_t)h * p.qs2 + dd;
      const double x = load_elem(p.q_cur, idx, p.esize);
      const double y = load_elem(p.q_prev, idx, p.esize);
      dot = fma(x, y, dot);
      nc = fma(x, x, nc);
      np = fma(y, y, np);
    }
  }
  red[t] = dot;
  red[nt + t] = nc;
  red[2 * nt + t] = np;
  __syncthreads();
  for (int s = nt / 2; s > 0; s >>= 1) {
    if (t < s) {
      red[t] += red[t + s];
      red[nt + t] += red[nt + t + s];
      red[2 * nt + t] += red[2 * nt + t + s];
    }
    __syncthreads();
  }
  if (t != 0) return;
  const int64_t bh = (int64_t)b * p.hq + h;
  double* part = p.ws_dbl + (bh * p.chunks + c) * 3;
  st_agent(part + 0, red[0]);
  st_agent(part + 1, red[nt]);
  st_agent(part + 2, red[2 * nt]);
  stores_done();  // partials acknowledged before the ticket
  int32_t* ticket = p.ws_int + bh;
  const int tk = atomicAdd(ticket, 1);
  if (tk != p.chunks - 1) return;
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
  st_agent(p.decision + bh, dec);
  if (p.ready) {
    stores_done();
    for (int c = 0; c < kReadyCopies; ++c) atomicAdd(p.ready + c * p.ready_stride + b, 1);
  }
}

// Gate workgroup wg of a grid of gate_grid(p) workgroups (count modes:
// position group fastest, then sequence; cosine: chunk, head, sequence); lds is scratch of
// at least 3 * blockDim.x doubles.  MULTI: the count modes may take several
// positions per workgroup (p.pos_per_wg); otherwise p.pos_per_wg must be 1.
template <bool MULTI>
__device__ __forceinline__ void run(const GateParams& p, int wg, void* lds) {
  if (p.mode != BA_GATE_COSINE) {
    if (p.vec16)
      count_body<u32x4, MULTI>(p, wg, lds);
    else if (p.esize == 4)
      count_body<uint32_t, MULTI>(p, wg, lds);
    else
      count_body<uint16_t, MULTI>(p, wg, lds);
  } else {
    const int c = wg % p.chunks, h = (wg / p.chunks) % p.hq, b = wg / (p.chunks * p.hq);
    cos_body(p, c, h, b, static_cast<double*>(lds));
  }
}

// Wait until the ready word at `word` reaches target (count mode:
// kCountReady; cosine: hq), polling with agent-scope loads; returns the word
// read, or -1 after `limit` polls.
__device__ __forceinline__ int wait_ready(const int32_t* word, int target, int limit) {
  for (int n = 0; n < limit; ++n) {
    const int r = __builtin_amdgcn_readfirstlane(ld_agent(word));
    if (r >= target) return r;
    __builtin_amdgcn_s_sleep(2);
  }
  return -1;
}

// As wait_ready, but each lane waits for its own word (the lanes of a wave
// may poll different words): returns this lane's word, or -1 after `limit`
// polls.
__device__ __forceinline__ int wait_ready_lane(const int32_t* word, int target, int limit) {
  int r = -1;
  for (int n = 0; n < limit; ++n) {
    const int x = ld_agent(word);
    if (x >= target) {
      r = x;
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  return r;
}

}  // namespace gate
}  // namespace ba
