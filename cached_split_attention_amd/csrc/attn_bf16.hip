// bf16 matrix-core attention for gfx950: prefix (out-of-block) attention with
// split-KV, and in-block attention with the fused log-space merge.
//
// The computation is the split of FlashBlock (gist.science/es/paper/2602.05305,
// section 2, "Mecanismo Central"): each part yields an output A and its
// natural log-normaliser L = log Z; parts are combined by the log-space merge
// equation of the same section (also used here to combine key splits).
//
// Per wave (64 lanes, 32 query rows):
//   S^T = K Q^T     v_mfma_f32_32x32x16_bf16, A = K (32 keys x 16 dims) from
//                   LDS, B = Q^T held in registers.  Lane l owns query row
//                   l%32; its 16 accumulators per 32-key block are keys
//                   8j + 4(l/32) + i (j, i = 0..3).
//   softmax         online, base 2 (scale*log2(e) folded into one FMA).  The
//                   reference max is only moved when some row's max grew by
//                   more than 2^8 (then all rows rescale), so most tiles skip
//                   the rescale of the output accumulators.  The max is shared
//                   by the two lane halves with one v_permlane32_swap per
//                   tile; row sums stay per half until the end.
//   O^T += V^T P^T  A = V^T (32 dims x 16 keys) gathered from row-major V in
//                   LDS by two ds_read_b64_tr_b16 (each 16-lane group reads a
//                   4-key x 16-dim block and receives it transposed), B = P^T
//                   straight from the S^T accumulators (8 consecutive
//                   accumulators = one 16-key step), so P never leaves
//                   registers.
// Staging: K and V tiles go from HBM to LDS with global_load_lds_dwordx4
// (no register round trip) into a ring of stages; a tile is waited for with
// s_waitcnt vmcnt and a workgroup barrier, so later tiles stay in flight
// while one is consumed.  Rows of K and V are 2*d bytes; their 16-byte chunks
// are XOR-swizzled by row so that both the 32-row K reads (ds_read_b128) and
// the 4-row V transpose reads hit distinct banks.
//
// Two workgroup shapes:
//   attn_bf16_kernel  RW row-waves x KW key-waves, one barrier per tile; key
//                     wave kg takes keys [kg*KT, (kg+1)*KT) of each tile and
//                     the key-waves' partial results are merged through LDS
//                     at the end.  Serves short and medium row counts.
//   attn_pp_kernel    eight waves over 256 rows in two groups of four that
//                     alternate between a matrix phase (P.V of the previous
//                     tile, then the scores of the next) and a vector phase
//                     (softmax of those scores), half a tile apart: while one
//                     group's wave on a SIMD issues MFMAs the other's issues
//                     the exponentials, so the matrix cores are not left idle
//                     during the softmax.  Serves long row counts.
// Work mapping: workgroups i and j of a launch run on the same XCD exactly
// when i = j (mod 8) (which XCD takes class 0 rotates between launches).
// Work items are groups (key split, sequence, KV head), split fastest,
// each with its row tiles; group g goes to XCD class g % 8 and its row
// tiles (which read the same K/V tiles) to consecutive workgroups of that
// class, so their re-reads hit that XCD's
// L2, while the groups of any subset of sequences or heads -- what a gated
// step recomputes -- spread over all XCDs.

#include <math.h>

#include <algorithm>
#include <atomic>

#include "ba_internal.h"
#include "gate_body.h"

namespace ba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kRescaleSlack = 8.0f;  // log2 units the reference max may lag
constexpr int kXcds = 8;

// IEEE maximum (NaN-propagating): maps to v_maximum3_f32 without the operand
// canonicalisation the C fmaxf needs.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Max over the score accumulators of MB 32-key blocks, as four independent
// chains of 3-input maxima.
template <int MB>
__device__ __forceinline__ float tile_max(const f32x16 (&s)[MB]) {
  float m[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const int c = (e >> 1) & 3;
      m[c] = vmax(vmax(m[c], s[mb][e]), s[mb][e + 1]);
    }
  return vmax(vmax(m[0], m[1]), vmax(m[2], m[3]));
}

__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  f32x2 x = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(x, bf16x2));
}

// 16 bytes from global memory straight into LDS: lane l's bytes land at
// lds_base + 16*l (M0 holds the wave-uniform base).  Written as asm so the
// compiler does not make every later LDS read wait for all DMA in flight;
// completion is tracked explicitly with s_waitcnt vmcnt.
__device__ __forceinline__ void dma16(const void* gsrc, unsigned lds_base) {
  const unsigned base = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "s"(base) : "memory");
}

// As dma16, from a wave-uniform base plus a per-lane 32-bit byte offset (the
// base is read from the first lane, so it lives in scalar registers).
// NT: the load is marked nontemporal (data read once).
template <bool NT = false>
__device__ __forceinline__ void dma16_s(const void* sbase, unsigned voff, unsigned lds_base) {
  const unsigned base = __builtin_amdgcn_readfirstlane(lds_base);
  // (readfirstlane returns int: each half goes through unsigned, so the low
  // half is zero-extended, not sign-extended, into the 64-bit address)
  const uint64_t a = reinterpret_cast<uint64_t>(sbase);
  const uint64_t lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)a);
  const uint64_t hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  const uint64_t su = lo | (hi << 32);
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(su), "s"(base) : "memory");
  else
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(su), "s"(base) : "memory");
}

// Wait until at most N vector-memory operations of this wave are in flight,
// then barrier the workgroup.  The memory clobber keeps the compiler from
// moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Wait for every vector-memory load of this wave, through the compiler's own
// s_waitcnt (vmcnt 0, other counters untouched), so the compiler knows the
// Q operand loads issued before it are complete.  Without it the compiler
// cannot prove that inside the tile loop, and makes the first score MFMA of
// every tile wait for vmcnt(0), which also waits out every K/V tile the
// ring has in flight.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// As wait_barrier, also draining this wave's LDS reads first, with nothing
// scheduled across it: a phase boundary of the alternating kernel.
template <int N>
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// 16-byte chunk swizzle of a K/V row in LDS (d = 128: 16 chunks, 256 bytes =
// one sweep of the 64 banks).  Swapping the two 2-bit halves of the row's low
// nibble makes (a) the 16 rows one ds_read_b128 phase reads at the same chunk
// land on 16 distinct chunks and (b) the 4 rows of a transposed V read land
// in 4 distinct 64-byte bank groups.
template <int D>
__device__ __forceinline__ int swz(int row) {
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((row & 3) << 1);
}

// DMA of K/V iteration tiles (KTILE keys) into LDS, shared by the NW waves of
// a workgroup: wave w fetches 1 KB blocks w*BPW .. w*BPW+BPW-1 of the K tile
// and of the V tile.  Lane l of a block writes row blk*RPB + l/CPR, chunk slot
// l%CPR, which holds source chunk (l%CPR) ^ swz(row).  A full tile is fetched
// from the tile's scalar base plus fixed per-lane byte offsets; the tail tile
// clamps keys past the range to the last valid key (finite data; their scores
// are masked).  With STREAM and `once` (a single row tile per (sequence, KV
// head), so each tile is read by one work item only) the full-tile loads
// are marked nontemporal: the stream then does not displace lines that are read again
// (LLaDA-like step 10.6 -> 10.1 us, multi-branch varlen step 139 -> 133-134
// us).  With several row tiles each tile is read once per row tile and the
// L2 serves the repeats (the video-like pass is 2 % slower with the mark).
template <int D, int NW, int KTILE, bool STREAM = false>
struct TileDma {
  static constexpr int ROWB = D * 2;
  static constexpr int CPR = D / 8;
  static constexpr int RPB = 1024 / ROWB;
  static constexpr int TILE_B = KTILE * ROWB;
  static constexpr int NBLK = TILE_B / 1024;
  static constexpr int BPW = NBLK / NW;
  static constexpr int OPS = 2 * BPW;  // vector-memory operations per wave per tile
  static_assert(NBLK % NW == 0 && BPW >= 1, "tile must split evenly into per-wave DMA blocks");

  const uint16_t* kptr;
  const uint16_t* vptr;
  int64_t ks1, vs1;
  int ke, w, l_row, l_slot;
  bool fast;
  unsigned koffs[BPW], voffs[BPW];
  bool once;

  __device__ __forceinline__ TileDma(const uint16_t* kp, const uint16_t* vp, int64_t ks, int64_t vs, int kend,
                                     int wave, int lane, bool read_once = false)
      : kptr(kp), vptr(vp), ks1(ks), vs1(vs), ke(kend), w(wave), l_row(lane / CPR), l_slot(lane % CPR),
        once(STREAM && read_once) {
    fast = (int64_t)KTILE * (ks1 > vs1 ? ks1 : vs1) * 2 < (1LL << 31);
#pragma unroll
    for (int u = 0; u < BPW; ++u) {
      const int row = (w * BPW + u) * RPB + l_row;
      const int c = l_slot ^ swz<D>(row);
      koffs[u] = fast ? (unsigned)((row * ks1 + c * 8) * 2) : 0u;
      voffs[u] = fast ? (unsigned)((row * vs1 + c * 8) * 2) : 0u;
    }
  }

  __device__ __forceinline__ void issue(int t0, unsigned kdst, unsigned vdst) const {
    if (fast && t0 + KTILE <= ke) {
      const uint16_t* kt = kptr + (int64_t)t0 * ks1;
      const uint16_t* vt = vptr + (int64_t)t0 * vs1;
      if (STREAM && once) {
#pragma unroll
        for (int u = 0; u < BPW; ++u) {
          const int blk = w * BPW + u;
          dma16_s<true>(kt, koffs[u], kdst + blk * 1024);
          dma16_s<true>(vt, voffs[u], vdst + blk * 1024);
        }
      } else {
#pragma unroll
        for (int u = 0; u < BPW; ++u) {
          const int blk = w * BPW + u;
          dma16_s(kt, koffs[u], kdst + blk * 1024);
          dma16_s(vt, voffs[u], vdst + blk * 1024);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < BPW; ++u) {
        const int blk = w * BPW + u;
        const int row = blk * RPB + l_row;
        const int c = l_slot ^ swz<D>(row);
        const int j = min(t0 + row, ke - 1);
        dma16(kptr + (int64_t)j * ks1 + c * 8, kdst + blk * 1024);
        dma16(vptr + (int64_t)j * vs1 + c * 8, vdst + blk * 1024);
      }
    }
  }
};

// Per-lane LDS byte offsets (within a stage) of the MFMA operands of a wave
// whose keys start at row k0 of the tile.  Key-block and 16-key-step offsets
// are multiples of 16 rows, leave the swizzle unchanged and go into the
// instructions' immediate offsets (the 16-bit mask tells the compiler the
// base is non-negative, which it needs before it folds a constant into a DS
// offset).
template <int D>
struct OperandOffsets {
  static constexpr int ROWB = D * 2;
  unsigned kro[D / 16];     // K (A of S^T): row k0 + lr, chunk 2*ks + hf
  unsigned vro[D / 32][2];  // V (A of O^T, transposed read)
  __device__ __forceinline__ OperandOffsets(int k0, int lane) {
    const int lr = lane & 31, hf = lane >> 5;
    {
      const int row = k0 + lr;
      const int sw = swz<D>(row);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) kro[ks] = (unsigned)(row * ROWB + (((2 * ks + hf) ^ sw) << 4)) & 0xffffu;
    }
    // 16-lane group tq covers dims db*32 + (tq%2)*16 .. +15; source lane ts
    // addresses key row k0 + 4*hf + ts/4 (+8 for the upper half of a 16-key
    // step), dims +4*(ts%4) .. +3, i.e. chunk 4db + 2(tq%2) + (ts%4)/2, half ts%2.
    const int tq = lane >> 4, ts = lane & 15;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int row = k0 + 8 * hi + 4 * hf + (ts >> 2);
        const int c = 4 * db + 2 * (tq & 1) + ((ts & 3) >> 1);
        vro[db][hi] = (unsigned)(row * ROWB + ((c ^ swz<D>(row)) << 4) + 8 * (ts & 1)) & 0xffffu;
      }
  }
};

// S^T (MB 32-key blocks) = K Q^T for the keys of one stage.
template <int D, int MB>
__device__ __forceinline__ void score_mfma(f32x16 (&s)[MB], const unsigned char* sK, const OperandOffsets<D>& off,
                                           const bf16x8 (&qf)[D / 16]) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) s[mb] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sK + off.kro[ks] + mb * 32 * (2 * D));
      s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[mb], 0, 0, 0);
    }
}

// O^T += V^T P^T for MB 32-key blocks; P packed as bf16, [block][16-key half].
template <int D, int MB>
__device__ __forceinline__ void pv_mfma(f32x16 (&o)[D / 32], const u32x4 (&pk)[MB][2], const unsigned char* sV,
                                        const OperandOffsets<D>& off) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const bf16x8 pf = __builtin_bit_cast(bf16x8, pk[mb][h2]);
      const int kofs = (mb * 32 + 16 * h2) * (2 * D);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(sV + off.vro[db][0] + kofs));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(sV + off.vro[db][1] + kofs));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[db], 0, 0, 0);
      }
    }
}

// A matrix phase of the alternating kernel: O^T += V^T P^T for the previous
// tile (MB blocks), then S^T = K Q^T for the next, as one stream of 2*MB*DB
// + MB*KS MFMAs whose LDS operand reads run PF MFMAs ahead of their use
// (a rotating set of PF fragments), so the read latency hides behind the
// MFMAs already issued instead of stalling each one.
template <int D, int MB, int PF>
__device__ __forceinline__ void matrix_phase(f32x16 (&o)[D / 32], const u32x4 (&pk)[MB][2], const unsigned char* sV,
                                             f32x16 (&s)[MB], const unsigned char* sK, const OperandOffsets<D>& off,
                                             const bf16x8 (&qf)[D / 16]) {
  constexpr int DB = D / 32, KS = D / 16;
  constexpr int NPV = MB * 2 * DB;    // P.V MFMAs: (block, 16-key half, 32-dim block)
  constexpr int NS_ = KS * MB;        // score MFMAs: (k-step, block)
  constexpr int N = NPV + NS_;
  bf16x8 frag[PF];
  auto read = [&](int i) -> bf16x8 {
    if (i < NPV) {
      const int mb = i / (2 * DB), h2 = (i / DB) % 2, db = i % DB;
      const int kofs = (mb * 32 + 16 * h2) * (2 * D);
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(sV + off.vro[db][0] + kofs));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(sV + off.vro[db][1] + kofs));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    const int j = i - NPV, ks = j / MB, mb = j % MB;
    return *reinterpret_cast<const bf16x8*>(sK + off.kro[ks] + mb * 32 * (2 * D));
  };
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) s[mb] = f32x16{};
#pragma unroll
  for (int i = 0; i < PF; ++i) frag[i] = read(i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    // each step (next read, this MFMA) stays in place: the scheduler would
    // otherwise sink the reads next to their MFMAs and expose their latency
    __builtin_amdgcn_sched_barrier(0);
    const bf16x8 a = frag[i % PF];
    if (i + PF < N) frag[i % PF] = read(i + PF);
    if (i < NPV) {
      const int mb = i / (2 * DB), h2 = (i / DB) % 2, db = i % DB;
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, pk[mb][h2]), o[db], 0, 0, 0);
    } else {
      const int j = i - NPV, ks = j / MB, mb = j % MB;
      s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[mb], 0, 0, 0);
    }
  }
}

// Online softmax of one tile's scores (MB blocks starting at key g0; keys at
// or past ke are masked): moves the reference max if needed (rescaling O and
// the running sum), turns the scores into P = 2^(s*c2 - m) in place, adds
// them to the running sum and packs them as bf16 for P.V.
template <int D, int MB>
__device__ __forceinline__ void softmax_tile(f32x16 (&s)[MB], u32x4 (&pk)[MB][2], f32x16 (&o)[D / 32], float& m_run,
                                             float& l_run, float c2, int g0, int ke, int hf) {
  if (g0 + MB * 32 > ke) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = g0 + mb * 32 + 8 * (e >> 2) + 4 * hf + (e & 3);
        if (key >= ke) s[mb][e] = -INFINITY;
      }
  }
  const float mx = pair_max(tile_max(s)) * c2;
  if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleSlack)) {
    const float m_new = vmax(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
    m_run = m_new;
  }
  float ps = 0.0f;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pv = __builtin_amdgcn_exp2f(fmaf(s[mb][e], c2, -m_run));
      s[mb][e] = pv;
      ps += pv;
    }
  l_run += ps;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int q = 0; q < 4; ++q) pk[mb][h2][q] = pack_bf16(s[mb][8 * h2 + 2 * q], s[mb][8 * h2 + 2 * q + 1]);
}

// The merge equation for one (row, head) entry: the weights of its two
// parts and the merged log-normaliser; a part with L = -inf weighs nothing,
// and both -inf give weights 0 and L = -inf.  The combine pass and the fused
// merge of the in-block kernels both go through these two functions, so
// they round alike.
struct MergeWeights {
  float w1, w2, l;
};
__device__ __forceinline__ MergeWeights merge_weights(float l1, float l2) {
  const float mm = fmaxf(l1, l2);
  MergeWeights r{0.0f, 0.0f, -INFINITY};
  if (mm != -INFINITY) {
    const float e1 = __builtin_amdgcn_exp2f((l1 - mm) * kLog2e);
    const float e2 = __builtin_amdgcn_exp2f((l2 - mm) * kLog2e);
    const float den = e1 + e2;
    const float rden = 1.0f / den;
    r.w1 = e1 * rden;
    r.w2 = e2 * rden;
    r.l = mm + __logf(den);
  }
  return r;
}
__device__ __forceinline__ float merge_elem(const MergeWeights& w, float x1, float x2) {
  return fmaf(w.w1, x1, w.w2 * x2);
}

// Where one lane's query row lives and what it writes.
struct RowOut {
  int64_t orow;    // output row (packed row for varlen, else the dense row)
  int64_t prow;    // b*max_q + i (split partials are laid out dense, by row index)
  int h;           // query head
  int hf;          // lane half: dims 8j + 4*hf .. +3 of each 32-dim block
  int split;
};

// Epilogue: normalises the accumulators and writes, by mode, the split
// partial, the final prefix result, or the in-block result with the fused
// log-space merge against the cached prefix result.
template <int D, bool PREFETCH>
__device__ __forceinline__ void write_result(const AttnParams& p, int mode, bool writer, const RowOut& ro,
                                             const f32x16 (&o)[D / 32], float m_run, float l_tot,
                                             const f32x4* cache_a, float cache_l) {
  constexpr int DB = D / 32;
  const int hf = ro.hf;
  const bool has = l_tot > 0.0f;
  const float inv = has ? 1.0f / l_tot : 0.0f;
  const float L = has ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  const int64_t oe = ro.orow * p.hq + ro.h;

  if (mode == kPrefixPartial) {
    // This split's partial result (normalised A and its L); the combine
    // kernel merges the splits.
    if (writer) {
      const int64_t n_entries = (int64_t)p.n_seq * p.max_q * p.hq;
      const int64_t ve = (int64_t)ro.split * n_entries + ro.prow * p.hq + ro.h;
      float* a = p.ws_a + ve * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 val = {o[db][4 * j] * inv, o[db][4 * j + 1] * inv, o[db][4 * j + 2] * inv,
                       o[db][4 * j + 3] * inv};
          *reinterpret_cast<f32x4*>(a + db * 32 + 8 * j + 4 * hf) = val;
        }
      if (hf == 0) p.ws_l[ve] = L;
    }
    return;
  }

  if (!writer) return;

  if (mode == kPrefixFinal) {
    float* a = p.a + oe * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 val = {o[db][4 * j] * inv, o[db][4 * j + 1] * inv, o[db][4 * j + 2] * inv,
                     o[db][4 * j + 3] * inv};
        *reinterpret_cast<f32x4*>(a + db * 32 + 8 * j + 4 * hf) = val;
      }
    if (hf == 0) p.l[oe] = L;
    return;
  }

  // In-block attention: optional A_in/L_in, optional fused merge with the cache.
  if (p.a) {
    float* a = p.a + oe * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 val = {o[db][4 * j] * inv, o[db][4 * j + 1] * inv, o[db][4 * j + 2] * inv,
                     o[db][4 * j + 3] * inv};
        *reinterpret_cast<f32x4*>(a + db * 32 + 8 * j + 4 * hf) = val;
      }
  }
  if (p.l && hf == 0) p.l[oe] = L;
  if (p.a_cache) {
    float lc;
    if constexpr (PREFETCH) lc = cache_l; else lc = p.l_cache[oe];
    // cache first, in-block part second, from the normalised A_in as stored
    const MergeWeights mw = merge_weights(lc, L);
    if (p.a_full) {
      const float* ac = p.a_cache + oe * D;
      float* af = p.a_full + oe * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c0 = db * 32 + 8 * j + 4 * hf;
          f32x4 cv;
          if constexpr (PREFETCH) cv = cache_a[db * 4 + j]; else cv = *reinterpret_cast<const f32x4*>(ac + c0);
          f32x4 val;
#pragma unroll
          for (int e = 0; e < 4; ++e) val[e] = merge_elem(mw, cv[e], o[db][4 * j + e] * inv);
          *reinterpret_cast<f32x4*>(af + c0) = val;
        }
    }
    if (p.l_full && hf == 0) p.l_full[oe] = mw.l;
  }
}

// Epilogue of the 256-row kernel (split partial, final prefix result,
// A_in/L_in, and the in-block result with the fused merge): the wave's normalised
// 32 x D block goes through its own LDS region (the ring is free once every
// tile is consumed), so that each global store writes whole rows (D floats
// contiguous) instead of a 32-byte piece of each of 32 rows.  In LDS, row rr
// keeps its 16-byte chunk c at position c ^ (rr mod chunks per row), so the
// row-owning writes and the chunk-owning reads both spread over the banks.
// The stores are nontemporal: the rows are read back by the next pass, not
// by this one (the GQA reuse step measured 20.9 -> 19.8 us with them).
// The fused merge reads the cached rows chunk by chunk the same way and
// writes A_full as whole rows (the video-like in-block call with the merge:
// 55.6-56.1 -> 50.4-50.8 us against the direct 32-byte stores).
// Every wave of the workgroup must call it (it starts with a barrier).
template <int D, bool MERGE>
__device__ __forceinline__ void write_result_staged(const AttnParams& p, int mode, bool writer, const RowOut& ro,
                                                    const f32x16 (&o)[D / 32], float m_run, float l_tot,
                                                    unsigned char* wave_lds) {
  constexpr int DB = D / 32;
  constexpr int CH = D / 4;          // 16-byte chunks per row
  constexpr int RPI = 64 / CH;       // rows per wave-wide store
  const int lane = (int)threadIdx.x & 63;
  const int lr = lane & 31, hf = ro.hf;
  const bool has = l_tot > 0.0f;
  const float inv = has ? 1.0f / l_tot : 0.0f;
  const float L = has ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  // destination entry of this lane's row (-1: not written)
  const int64_t n_entries = (int64_t)p.n_seq * p.max_q * p.hq;
  const bool partial = mode == kPrefixPartial;
  float* a_base = partial ? p.ws_a : p.a;
  float* l_base = partial ? p.ws_l : p.l;
  const int64_t ent = partial ? (int64_t)ro.split * n_entries + ro.prow * p.hq + ro.h : ro.orow * p.hq + ro.h;
  const int my_ent = writer ? (int)ent : -1;
  constexpr int NI = 32 / RPI;       // wave-wide stores per 32 rows
  const int cc = lane % CH;          // the chunk this lane stores

  wait_vmem_all();
  // In-block result with the fused merge: the cached prefix rows this lane
  // merges (the chunks it stores) are loaded first, all together, so their
  // latency hides behind the barrier and the staging below.
  const bool merge = MERGE && mode == kBlock && p.a_cache != nullptr;
  float lc[NI];
  f32x4 cv[NI];
  if constexpr (MERGE) if (merge) {
#pragma unroll
    for (int s = 0; s < NI; ++s) {
      const int e = __shfl(my_ent, RPI * s + lane / CH);
      lc[s] = e >= 0 ? p.l_cache[e] : -INFINITY;
      cv[s] = (e >= 0 && p.a_full) ? *reinterpret_cast<const f32x4*>(p.a_cache + (int64_t)e * D + 4 * cc)
                                   : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }
  __syncthreads();   // every wave is done with the ring
  f32x4* rowp = reinterpret_cast<f32x4*>(wave_lds + lr * (D * 4));
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = db * 8 + 2 * j + hf;
      rowp[c ^ (lr & (CH - 1))] = f32x4{o[db][4 * j] * inv, o[db][4 * j + 1] * inv, o[db][4 * j + 2] * inv,
                                        o[db][4 * j + 3] * inv};
    }
  if (a_base) {
#pragma unroll
    for (int s = 0; s < NI; ++s) {
      const int rr = RPI * s + lane / CH;
      const int e = __shfl(my_ent, rr);
      const f32x4 val = reinterpret_cast<const f32x4*>(wave_lds + rr * (D * 4))[cc ^ (rr & (CH - 1))];
      if (e >= 0) __builtin_nontemporal_store(val, reinterpret_cast<f32x4*>(a_base + (int64_t)e * D + 4 * cc));
    }
  }
  if (l_base && writer && hf == 0) l_base[ent] = L;
  if constexpr (MERGE) if (merge) {
    // the merge equation, cache first and in-block part second, from the
    // normalised A_in as staged (the same arithmetic as the direct epilogue)
#pragma unroll
    for (int s = 0; s < NI; ++s) {
      const int rr = RPI * s + lane / CH;
      const int e = __shfl(my_ent, rr);
      const float li = __shfl(L, rr);
      const MergeWeights mw = merge_weights(lc[s], li);
      if (e >= 0 && p.a_full) {
        const f32x4 val = reinterpret_cast<const f32x4*>(wave_lds + rr * (D * 4))[cc ^ (rr & (CH - 1))];
        f32x4 af;
#pragma unroll
        for (int k = 0; k < 4; ++k) af[k] = merge_elem(mw, cv[s][k], val[k]);
        __builtin_nontemporal_store(af, reinterpret_cast<f32x4*>(p.a_full + (int64_t)e * D + 4 * cc));
      }
      if (e >= 0 && p.l_full && cc == 0) p.l_full[e] = mw.l;
    }
  }
}

// Work item of a workgroup covering ROWS query rows: (sequence, KV head,
// row tile, key split) and the sequence's query/key ranges.
struct Item {
  int split, rt, b, kvh;
  int qbase, nq, kbase, nk;
  int row0, kb, ke, mode;
  bool valid;
};

// Work item group (key split, sequence, KV head; split fastest) of
// workgroup wg: groups are dealt to the XCDs in turn, each with its row
// tiles on consecutive workgroups of its XCD (workgroups whose numbers are
// congruent mod kXcds share an XCD).  A group past n_splits * n_seq * hkv
// is no work.
__device__ __forceinline__ int item_group(const AttnParams& p, int wg) {
  return (wg / kXcds / p.row_tiles) * kXcds + wg % kXcds;
}

// Workgroups of a part's grid: groups dealt to the XCDs in turn, each with
// its row tiles (item_group numbers them).
__host__ __device__ __forceinline__ int item_grid_size(const AttnParams& p) {
  const int n_groups = p.n_splits * p.n_seq * p.hkv;
  return kXcds * ((n_groups + kXcds - 1) / kXcds) * p.row_tiles;
}

template <int ROWS>
__device__ __forceinline__ Item decode_item(const AttnParams& p, int wg) {
  Item it{};
  const int j = wg / kXcds;
  const int g = item_group(p, wg);   // (split, sequence, KV head)
  it.valid = false;
  if (g >= p.n_splits * p.n_seq * p.hkv) return it;
  it.split = g % p.n_splits;
  it.rt = j % p.row_tiles;
  const int bz = g / p.n_splits;
  it.b = bz / p.hkv;
  it.kvh = bz - it.b * p.hkv;
  it.qbase = 0;
  it.nq = p.max_q;
  it.kbase = 0;
  it.nk = p.max_k;
  if (p.cu_q != nullptr) {
    it.qbase = p.cu_q[it.b];
    it.nq = min(max(p.cu_q[it.b + 1] - it.qbase, 0), p.max_q);   // (rows beyond max_q are ignored)
  }
  if (p.cu_k != nullptr) {
    it.kbase = p.cu_k[it.b];
    it.nk = p.cu_k[it.b + 1] - it.kbase;
  }
  const int R = p.group * it.nq;
  it.row0 = it.rt * ROWS;
  if (it.row0 >= R) return it;
  // the key range [kb, ke) counts keys, or list entries in key-block mode
  const int units = p.kblocks ? p.n_kblocks : it.nk;
  it.kb = it.split * p.chunk;
  // A sequence with no keys at all is finished by split 0 alone (A = 0,
  // L = -inf); otherwise splits past the end have nothing to do.
  it.mode = (p.mode == kPrefixPartial && units == 0) ? kPrefixFinal : p.mode;
  if (p.mode == kPrefixPartial && it.kb >= units && !(units == 0 && it.split == 0)) return it;
  it.ke = min(units, it.kb + p.chunk);
  it.valid = true;
  return it;
}

// Key-block list mode: this lane's entry of the workgroup's list range
// (entries kb + lane, lane < ke - kb <= 64), clamped into the sequence's
// blocks so that a bad index can only give a wrong result, never an access
// outside K/V.  Tile it starts at key readlane(entry, it) * kBlockKeys.
__device__ __forceinline__ int load_block_entry(const AttnParams& p, const Item& it, int lane) {
  if (!p.kblocks) return 0;
  const int64_t base = ((int64_t)it.b * p.hkv + it.kvh) * p.n_kblocks + it.kb;
  int e = lane < it.ke - it.kb ? p.kblocks[base + lane] : 0;
  const int last = (it.nk + kBlockKeys - 1) / kBlockKeys - 1;
  return min(max(e, 0), last);
}

// Reuse decision of (sequence b, query head h).  Read with agent-scope loads:
// the gate may have written it from another XCD earlier in the same launch.
__device__ __forceinline__ bool reused(const AttnParams& p, int b, int h) {
  return gate::ld_agent(p.decision + b * p.hq + h) != 0;
}

// True if some query head of rows [row0, row0+ROWS) needs its prefix
// attention recomputed.
template <int ROWS>
__device__ __forceinline__ bool any_recompute(const AttnParams& p, const Item& it) {
  const int R = p.group * it.nq;
  const int rlast = min(R, it.row0 + ROWS) - 1;
  bool any = false;
  for (int g = it.row0 / it.nq; g <= rlast / it.nq; ++g) any |= !reused(p, it.b, it.kvh * p.group + g);
  return any;
}

// A gated prefix workgroup of a launch that also runs the gate: wait until
// the gate has published sequence b's result.  One thread polls and the
// answer is shared through LDS, so every wave takes the same path.
// Returns 0: all heads of the workgroup are reused (nothing to do); 1: all
// recompute (count mode with M_b >= tau, or a wait that gave up, counted in
// *gave_up; the launch then writes split partials, which the combine pass
// applies only where the decision is 0); 2: the per-head decisions are
// written (cosine mode).
__device__ __forceinline__ int gate_ready(const AttnParams& p, int b) {
  __shared__ int s_r;
  if (threadIdx.x == 0) {
    const bool count = p.gate_mode != BA_GATE_COSINE;   // count or cumulative count
    const int32_t* word = p.ready + (int)(blockIdx.x % kReadyCopies) * p.ready_stride + b;
    const int r = gate::wait_ready(word, count ? gate::kCountReady : p.hq, p.spin_limit);
    int res;
    if (r < 0) {
      if (p.gave_up) atomicAdd(p.gave_up, 1);
      res = 1;
    } else if (count) {
      res = (r & (gate::kCountReady - 1)) < p.gate_tau ? 0 : 1;
    } else {
      res = 2;
    }
    s_r = res;
  }
  __syncthreads();
  return s_r;
}

// One work item of the row-wave/key-wave kernel: number wg of part p's
// grid.  Every wave of the workgroup returns from it together.
template <int D, int RW, int KW, int KT, int ST, bool GATE>
__device__ __forceinline__ void bf16_item(const AttnParams& p, const int wg, unsigned char* smem) {
  constexpr int NW = RW * KW;
  constexpr int KTILE = KW * KT;                 // keys per iteration tile
  // (nontemporal K/V streams where each tile is read once; the 256-row
  // kernel, bound by its matrix cores, keeps cached loads: the mark measured
  // 0.3 % slower on the GQA schedule there)
  using Dma = TileDma<D, NW, KTILE, true>;
  constexpr int TILE_B = Dma::TILE_B;            // bytes of one K (or V) tile
  constexpr int KS = D / 16;                     // MFMA k-steps over head dim
  constexpr int DB = D / 32;                     // 32-dim output blocks
  constexpr int MB = KT / 32;                    // 32-key blocks per key-wave
  static_assert(ST >= 2 && ST <= 4, "ring depth");
  constexpr int STAGE_B = 2 * TILE_B;
  constexpr int XSLOT = (DB * 16 + 2) * 64;      // floats per key-wave exchange slot
  const unsigned smem_base = (unsigned)(uintptr_t)smem;

  bool gated = p.decision != nullptr && p.mode != kBlock;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int rw = w % RW, kg = w / RW;
  const int lr = lane & 31, hf = lane >> 5;

  const Item itm = decode_item<RW * 32>(p, wg);
  if (!itm.valid) return;
  if constexpr (GATE) {
    if (gated && p.ready) {
      const int r = gate_ready(p, itm.b);
      if (r == 0) return;
      gated = r == 2;
    }
  }
  if (gated && !any_recompute<RW * 32>(p, itm)) return;
  const bool qvar = p.cu_q != nullptr && p.q_rows == nullptr;   // packed Q rows
  const bool kvar = p.cu_k != nullptr;
  const int G = p.group, nq = itm.nq, b = itm.b, kvh = itm.kvh, kb = itm.kb, ke = itm.ke;
  const int R = G * nq;

  // --- this lane's query row and its Q operand (B of S^T = K Q^T) ---
  const int r = itm.row0 + rw * 32 + lr;
  const bool rvalid = r < R;
  const int g = rvalid ? r / nq : 0;
  const int i = rvalid ? r - g * nq : 0;
  const int h = kvh * G + g;
  const int qi = (p.q_rows && rvalid) ? listed_row(p, b, itm.qbase + i) : i;   // dense position
  const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
      (qvar ? (int64_t)(itm.qbase + i) * p.qs1 : (int64_t)b * p.qs0 + (int64_t)qi * p.qs1) +
      (int64_t)h * p.qs2;
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 x = rvalid ? *reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * hf) : u32x4{0, 0, 0, 0};
    qf[ks] = __builtin_bit_cast(bf16x8, x);
  }

  const uint16_t* kptr = static_cast<const uint16_t*>(p.k) +
      (kvar ? (int64_t)itm.kbase * p.ks1 : (int64_t)b * p.ks0) + (int64_t)kvh * p.ks2;
  const uint16_t* vptr = static_cast<const uint16_t*>(p.v) +
      (kvar ? (int64_t)itm.kbase * p.vs1 : (int64_t)b * p.vs0) + (int64_t)kvh * p.vs2;
  // key-block list mode: tiles are the listed blocks (KTILE == kBlockKeys)
  const bool listed = p.kblocks != nullptr;
  const int entry = load_block_entry(p, itm, lane);
  const Dma dma(kptr, vptr, p.ks1, p.vs1, listed ? itm.nk : ke, w, lane, p.row_tiles == 1);
  auto issue_tile = [&](int t0, int st) {
    const unsigned kdst = smem_base + st * STAGE_B;
    dma.issue(t0, kdst, kdst + TILE_B);
  };

  // Single-wave workgroups serve small in-block problems, where the cache read
  // of the merge would otherwise be one more memory round trip after the
  // compute: fetch this lane's cached A_out/L_out now.
  constexpr bool kPrefetchCache = (NW == 1);
  f32x4 cache_a[kPrefetchCache ? 4 * DB : 1];
  float cache_l = 0.0f;
  if constexpr (kPrefetchCache) {
    if (p.mode == kBlock && p.a_cache && rvalid) {
      const int64_t ce = (qvar ? (int64_t)(itm.qbase + i) : (int64_t)b * p.max_q + qi) * p.hq + h;
      cache_l = p.l_cache[ce];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          cache_a[db * 4 + j] = *reinterpret_cast<const f32x4*>(p.a_cache + ce * D + db * 32 + 8 * j + 4 * hf);
    }
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.0f;
  const float c2 = p.scale_log2;
  const OperandOffsets<D> off(kg * KT, lane);

  auto compute_tile = [&](const unsigned char* sK, const unsigned char* sV, int g0, int g1) {
    f32x16 s[MB];
    u32x4 pk[MB][2];
    score_mfma<D, MB>(s, sK, off, qf);
    softmax_tile<D, MB>(s, pk, o, m_run, l_run, c2, g0, g1, hf);
    pv_mfma<D, MB>(o, pk, sV, off);
  };

  const int n_iter = listed ? ke - kb : (ke > kb) ? (ke - kb + KTILE - 1) / KTILE : 0;
  // first key and key bound of tile it
  auto tile_key = [&](int it) { return listed ? __builtin_amdgcn_readlane(entry, it) * KTILE : kb + it * KTILE; };
  auto tile_end = [&](int it) { return listed ? min(tile_key(it) + KTILE, itm.nk) : ke; };
#pragma unroll
  for (int s = 0; s < ST - 1; ++s)
    if (s < n_iter) issue_tile(tile_key(s), s);
  wait_vmem_all();

  // The loop is unrolled over the ring so each copy reads a fixed stage.
  for (int it0 = 0; it0 < n_iter; it0 += ST) {
#pragma unroll
    for (int st = 0; st < ST; ++st) {
      const int it = it0 + st;
      if (it < n_iter) {
        const int ahead = min(ST - 2, n_iter - 1 - it);   // tiles issued after this one
        if constexpr (ST == 2) {
          wait_barrier<0>();
        } else if constexpr (ST == 3) {
          if (ahead >= 1) wait_barrier<Dma::OPS>(); else wait_barrier<0>();
        } else {
          if (ahead >= 2) wait_barrier<2 * Dma::OPS>();
          else if (ahead == 1) wait_barrier<Dma::OPS>();
          else wait_barrier<0>();
        }
        if (it + ST - 1 < n_iter) issue_tile(tile_key(it + ST - 1), (st + ST - 1) % ST);
        const int g0 = tile_key(it) + kg * KT, g1 = tile_end(it);
        if (g0 < g1) compute_tile(smem + st * STAGE_B, smem + st * STAGE_B + TILE_B, g0, g1);
      }
    }
  }

  float l_tot = pair_sum(l_run);

  if constexpr (KW > 1) {
    wait_barrier<0>();
    float* xs = reinterpret_cast<float*>(smem);
    if (kg > 0) {
      float* slot = xs + ((kg - 1) * RW + rw) * XSLOT;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) slot[(db * 16 + e) * 64 + lane] = o[db][e];
      slot[(DB * 16) * 64 + lane] = m_run;
      slot[(DB * 16 + 1) * 64 + lane] = l_tot;
    }
    __syncthreads();
    if (kg == 0) {
      float mall = m_run;
#pragma unroll
      for (int q = 1; q < KW; ++q) mall = fmaxf(mall, xs[((q - 1) * RW + rw) * XSLOT + (DB * 16) * 64 + lane]);
      if (mall != -INFINITY) {
        const float a0 = __builtin_amdgcn_exp2f(m_run - mall);
        l_tot *= a0;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= a0;
#pragma unroll
        for (int q = 1; q < KW; ++q) {
          const float* slot = xs + ((q - 1) * RW + rw) * XSLOT;
          const float aq = __builtin_amdgcn_exp2f(slot[(DB * 16) * 64 + lane] - mall);
          l_tot += aq * slot[(DB * 16 + 1) * 64 + lane];
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[db][e] += aq * slot[(db * 16 + e) * 64 + lane];
        }
      }
      m_run = mall;
    }
  }

  bool writer = kg == 0 && rvalid;
  if (gated) writer = writer && !reused(p, b, h);
  const RowOut ro{qvar ? (int64_t)(itm.qbase + i) : (int64_t)b * p.max_q + qi, (int64_t)b * p.max_q + i, h, hf,
                  itm.split};
  // (the LDS-staged epilogue of the 256-row kernel measured slower here: the
  // LLaDA-like prefix pass took 21.2 us against 19.8)
  write_result<D, kPrefetchCache>(p, itm.mode, writer, ro, o, m_run, l_tot, cache_a, cache_l);
}

// A launch may carry two independent parts (the prefix and the in-block
// attention of one step): workgroups [0, grid0) run part p0, the rest p1.
// With GATE, the reuse gate gp runs first, in workgroups [0, grid_g), and
// the rest are numbered from there.
template <int D, int RW, int KW, int KT, int ST, bool DUAL, bool GATE>
__global__ void __launch_bounds__(64 * RW * KW)
    __attribute__((amdgpu_waves_per_eu(ST * 4 * KW * KT * D > 80 * 1024 ? 1 : 2)))
attn_bf16_kernel(const AttnParams p0, const AttnParams p1, int grid0, const GateParams gp, int grid_g) {
  constexpr int KTILE = KW * KT;
  constexpr int TILE_B = TileDma<D, RW * KW, KTILE>::TILE_B;
  constexpr int XSLOT = (D / 32 * 16 + 2) * 64;
  constexpr int SMEM_X = (KW > 1) ? (KW - 1) * RW * XSLOT * 4 : 0;
  constexpr int SMEM_R = ST * 2 * TILE_B;
  constexpr int SMEM = SMEM_R > SMEM_X ? SMEM_R : SMEM_X;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[SMEM];
  int bid = (int)blockIdx.x;
  if constexpr (GATE) {
    if (bid < grid_g) {
      gate::run<false>(gp, bid, smem);
      return;
    }
    bid -= grid_g;
  }
  // (two calls rather than one on a reference chosen between the two
  // parameter blocks, which would make the compiler copy both to scratch)
  if (DUAL && bid >= grid0)
    bf16_item<D, RW, KW, KT, ST, GATE>(p1, bid - grid0, smem);
  else
    bf16_item<D, RW, KW, KT, ST, GATE>(p0, bid, smem);
}

// One work item of the alternating-phase kernel: (key split, sequence, KV
// head, row tile) number wg of part p's grid.  gated: the part is gated by
// decisions (with p.ready: read through the gate's ready words; ready_r >= 0
// is the gate result already read).  Every wave of the workgroup returns
// from it together.
template <int D, int NS, bool GATE, bool MERGE = false>
__device__ __forceinline__ void pp_item(const AttnParams& p, const int wg, bool gated, const int ready_r,
                                        unsigned char* smem) {
  constexpr int NW = 8, ROWS = 256, KT = 64;
  constexpr int LOOK = NS - 2;   // tiles issued ahead of the one waited for
  static_assert(LOOK >= 1 && LOOK <= 3, "ring depth");
  using Dma = TileDma<D, NW, KT>;
  constexpr int TILE_B = Dma::TILE_B;
  constexpr int STAGE_B = 2 * TILE_B;
  constexpr int KS = D / 16, DB = D / 32, MB = KT / 32;
  const unsigned smem_base = (unsigned)(uintptr_t)smem;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int grp = w >> 2;
  const int lr = lane & 31, hf = lane >> 5;

  const Item itm = decode_item<ROWS>(p, wg);
  if (!itm.valid) return;
  if constexpr (GATE) {
    if (gated && p.ready) {
      const int r = ready_r >= 0 ? ready_r : gate_ready(p, itm.b);
      if (r == 0) return;
      gated = r == 2;
    }
  }
  if (gated && !any_recompute<ROWS>(p, itm)) return;
  const bool qvar = p.cu_q != nullptr && p.q_rows == nullptr;   // packed Q rows
  const bool kvar = p.cu_k != nullptr;
  const int G = p.group, nq = itm.nq, b = itm.b, kvh = itm.kvh, kb = itm.kb, ke = itm.ke;
  const int R = G * nq;

  const int r = itm.row0 + w * 32 + lr;
  const bool rvalid = r < R;
  const bool active = itm.row0 + w * 32 < R;   // wave has some valid row
  const int g = rvalid ? r / nq : 0;
  const int i = rvalid ? r - g * nq : 0;
  const int h = kvh * G + g;
  const int qi = (p.q_rows && rvalid) ? listed_row(p, b, itm.qbase + i) : i;   // dense position
  const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
      (qvar ? (int64_t)(itm.qbase + i) * p.qs1 : (int64_t)b * p.qs0 + (int64_t)qi * p.qs1) +
      (int64_t)h * p.qs2;
  // The wave's 32 Q rows go to LDS first, through the ring's stages 2 and 3
  // (free until tile 2 is issued), by DMA instructions that each copy RPI
  // whole rows: a lane-per-row register load would touch 32 rows' cache
  // lines per instruction.  Each row's 16-byte chunks are XOR-placed by row,
  // so the operand reads below (chunk 2 ks + hf of row lr) hit distinct
  // banks.  A wave reads back only the rows it copied itself.
  constexpr int CH = D / 8, RPI = 64 / CH;
  const int q_lds_off = 2 * STAGE_B + w * (64 * D);
  if (active) {
    const uint64_t qa = reinterpret_cast<uint64_t>(qrow);
    const int qlo = (int)(unsigned)qa, qhi = (int)(unsigned)(qa >> 32), qv = rvalid ? 1 : 0;
    const int slot = lane & (CH - 1);
#pragma unroll
    for (int j = 0; j < 32 / RPI; ++j) {
      const int rr = RPI * j + lane / CH;
      const uint64_t a = (uint64_t)(unsigned)__shfl(qlo, rr) | ((uint64_t)(unsigned)__shfl(qhi, rr) << 32);
      if (__shfl(qv, rr))
        dma16(reinterpret_cast<const uint16_t*>(a) + 8 * (slot ^ (rr & (CH - 1))), smem_base + q_lds_off + j * 1024);
    }
  }

  const uint16_t* kptr = static_cast<const uint16_t*>(p.k) +
      (kvar ? (int64_t)itm.kbase * p.ks1 : (int64_t)b * p.ks0) + (int64_t)kvh * p.ks2;
  const uint16_t* vptr = static_cast<const uint16_t*>(p.v) +
      (kvar ? (int64_t)itm.kbase * p.vs1 : (int64_t)b * p.vs0) + (int64_t)kvh * p.vs2;
  // key-block list mode: tiles are the listed blocks (KT == kBlockKeys)
  const bool listed = p.kblocks != nullptr;
  const int entry = load_block_entry(p, itm, lane);
  auto tile_key = [&](int u) { return listed ? __builtin_amdgcn_readlane(entry, u) * KT : kb + u * KT; };
  auto tile_end = [&](int u) { return listed ? min(tile_key(u) + KT, itm.nk) : ke; };
  const Dma dma(kptr, vptr, p.ks1, p.vs1, listed ? itm.nk : ke, w, lane);
  auto issue_tile = [&](int u) {
    const unsigned kdst = smem_base + (u % NS) * STAGE_B;
    dma.issue(tile_key(u), kdst, kdst + TILE_B);
  };

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.0f;
  const float c2 = p.scale_log2;
  const OperandOffsets<D> off(0, lane);
  f32x16 s[MB];
  u32x4 pk[MB][2];

  // Each wave runs the same phase sequence
  //   M0: S(0) | V0: softmax(0) | M1: P.V(0), S(1) | V1 | ... | Mn: P.V(n-1)
  // (2n+1 phases, each opened by a barrier); group 1 passes one extra
  // barrier first and group 0 one extra at the end, so group 1 runs one
  // phase behind.  At every even workgroup phase 2v all waves wait for tile
  // v and issue tile v+2; for group 0 these are the barriers opening its
  // matrix phases, for group 1 those opening its vector phases.
  const int n = listed ? ke - kb : (ke > kb) ? (ke - kb + KT - 1) / KT : 0;
  auto even_barrier = [&](int v) {
    const int later = min(LOOK - 1, n - 1 - v);   // tiles issued after tile v
    if (later >= 2) phase_barrier<2 * Dma::OPS>();
    else if (later == 1) phase_barrier<Dma::OPS>();
    else phase_barrier<0>();
    if (v + LOOK < n) issue_tile(v + LOOK);
  };
#pragma unroll
  for (int t = 0; t < LOOK; ++t)
    if (t < n) issue_tile(t);
  wait_vmem_all();
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // (orders the LDS reads below after the copies)
  bf16x8 qf[KS];
  {
    const unsigned char* qw = smem + q_lds_off + lr * (2 * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(qw + 16 * ((2 * ks + hf) ^ (lr & (CH - 1))));
      qf[ks] = __builtin_bit_cast(bf16x8, rvalid ? x : u32x4{0, 0, 0, 0});
    }
  }
  if (grp) even_barrier(0);
  if (grp) phase_barrier<63>(); else even_barrier(0);
  if (active && n > 0) score_mfma<D, MB>(s, smem, off, qf);
  for (int u = 0; u < n; ++u) {
    if (grp) even_barrier(u + 1); else phase_barrier<63>();
    if (active) softmax_tile<D, MB>(s, pk, o, m_run, l_run, c2, tile_key(u), tile_end(u), hf);
    if (grp) phase_barrier<63>(); else even_barrier(u + 1);
    // (after the last tile the scores are computed from a stale stage and
    // never used: one branch-free block keeps the accumulators in place).
    // The matrix phase runs at raised wave priority, so that on a SIMD the
    // MFMA wave's instructions go first when both waves are ready (2-3 % on
    // the video-like and GQA shapes).
    __builtin_amdgcn_s_setprio(3);
    if (active)
      matrix_phase<D, MB, 4>(o, pk, smem + (u % NS) * STAGE_B + TILE_B, s, smem + ((u + 1) % NS) * STAGE_B, off,
                             qf);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  }
  if (!grp) phase_barrier<63>();

  const float l_tot = pair_sum(l_run);
  bool writer = rvalid;
  if (gated) writer = writer && !reused(p, b, h);
  const RowOut ro{qvar ? (int64_t)(itm.qbase + i) : (int64_t)b * p.max_q + qi, (int64_t)b * p.max_q + i, h, hf,
                  itm.split};
  // (the fused merge belongs to the stand-alone in-block call, whose launch
  // is the plain one-part kernel; the other launches keep its code out)
  if constexpr (MERGE)
    write_result_staged<D, true>(p, itm.mode, writer, ro, o, m_run, l_tot, smem + w * (32 * D * 4));
  else if (itm.mode == kBlock && p.a_cache)
    write_result<D, false>(p, itm.mode, writer, ro, o, m_run, l_tot, nullptr, 0.0f);
  else
    write_result_staged<D, false>(p, itm.mode, writer, ro, o, m_run, l_tot, smem + w * (32 * D * 4));
}

// Alternating-phase kernel: 8 waves, 256 query rows, 64-key tiles in an
// NS-stage ring.  Group grp (waves 4*grp .. 4*grp+3, rows 128*grp .. +127)
// alternates matrix phases (O += P(u-1) V(u-1), then S(u) = K(u) Q^T) and
// vector phases (softmax of S(u) into P(u)), group 1 one phase behind group
// 0, so at every workgroup phase one group is in its matrix phase and the
// other in its vector phase; waves w and w+4 share a SIMD.  Every wave passes
// the same 2n+2 barriers (n tiles).  Tile u is waited for at workgroup phase
// 2u and last read (as V by group 1) in phase 2u+3, so its stage can take
// tile u+NS from phase 2u+4 on: at phase 2u tile u+NS-2 is issued, and tiles
// u+1 .. u+NS-3 may still be in flight.
template <int D, int NS, bool DUAL, bool GATE, bool PERSIST = false>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_pp_kernel(const AttnParams p0, const AttnParams p1, int grid0, const GateParams gp, int grid_g) {
  constexpr int STAGE_B = 2 * TileDma<D, 8, 64>::TILE_B;   // a K and a V tile of 64 keys
  __shared__ __attribute__((aligned(1024))) unsigned char smem[NS * STAGE_B];

  int bid = (int)blockIdx.x;
  if constexpr (GATE) {
    if (bid < grid_g) {
      gate::run<true>(gp, bid, smem);
      return;
    }
    bid -= grid_g;
  }
  const bool second = DUAL && bid >= grid0;
  const int wg = second ? bid - grid0 : bid;
  if constexpr (PERSIST) {
    static_assert(GATE && DUAL, "the persistent prefix part belongs to a gated fused launch");
    if (second) {
      // Persistent gated prefix part of a count-gated step: prefix workgroup
      // wg of p1.persist takes work items wg, wg + persist, ... of the part's
      // grid.  Lane k of wave 0 reads the gate result of the k-th of them
      // (up to 64 at once), and the workgroup computes those whose sequence
      // recomputes (all of their heads).  The items of one sequence are
      // consecutive, so a step that recomputes a few sequences spreads them
      // over many workgroups, and a step that reuses everything costs each
      // workgroup one round of reads.
      __shared__ unsigned long long s_need;
      const int stride = p1.persist;
      const int n_items = item_grid_size(p1);
      for (int k0 = wg; k0 < n_items; k0 += 64 * stride) {
        if (threadIdx.x < 64) {
          const int v = k0 + (int)threadIdx.x * stride;
          bool need = false;
          if (v < n_items) {
            const int g = item_group(p1, v);
            if (g < p1.n_splits * p1.n_seq * p1.hkv) {
              const int32_t* word =
                  p1.ready + (int)(blockIdx.x % kReadyCopies) * p1.ready_stride + g / p1.n_splits / p1.hkv;
              const int r = gate::wait_ready_lane(word, gate::kCountReady, p1.spin_limit);
              if (r < 0) {
                if (p1.gave_up) atomicAdd(p1.gave_up, 1);
                need = true;   // (split partials: the combine pass applies the decision)
              } else {
                need = (r & (gate::kCountReady - 1)) >= p1.gate_tau;
              }
            }
          }
          const unsigned long long bits = __builtin_amdgcn_ballot_w64(need);
          if (threadIdx.x == 0) s_need = bits;
        }
        __syncthreads();
        unsigned long long m = s_need;
        __syncthreads();   // (s_need is rewritten by the next chunk)
        while (m) {
          const int k = __builtin_ctzll(m);
          m &= m - 1;
          pp_item<D, NS, GATE>(p1, k0 + k * stride, false, 1, smem);
          __syncthreads();   // the next item's DMA reuses the ring stages
        }
      }
      return;
    }
  }
  // A gated prefix workgroup reads its sequence's gate result first, from
  // the prefix part's parameters alone (few dependent kernel-argument
  // loads), and leaves at once when the whole sequence is reused: most
  // prefix workgroups of a reuse step do only this.
  int ready_r = -1;
  if constexpr (GATE) {
    if (second && p1.decision != nullptr && p1.ready != nullptr && p1.mode != kBlock) {
      const int g = item_group(p1, wg);
      if (g >= p1.n_splits * p1.n_seq * p1.hkv) return;
      ready_r = gate_ready(p1, g / p1.n_splits / p1.hkv);
      if (ready_r == 0) return;
    }
  }

  // (two calls rather than one on a reference chosen between the two
  // parameter blocks, which would make the compiler copy both to scratch)
  if (second)
    pp_item<D, NS, GATE>(p1, wg, p1.decision != nullptr && p1.mode != kBlock, ready_r, smem);
  else
    pp_item<D, NS, GATE, !DUAL && !GATE>(p0, wg, p0.decision != nullptr && p0.mode != kBlock, ready_r, smem);
}

// Compute units of the current device (looked up once per device; threads
// that race on the first lookup store the same value).
int device_cus() {
  static std::atomic<int> cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// One entry of the combine: where it lives and what its first memory round
// trip brought (the in-block part and, speculatively, the cached prefix
// result, loaded together with the decision).
struct CombineEntry {
  int64_t oo;     // output entry (row * hq + head); -1: nothing to do
  int64_t e;      // dense entry (split partials are laid out by it)
  int units;      // keys, or listed key blocks
  bool fresh;     // the prefix was recomputed: combine the split partials
  float li, l_c;
  f32x4 ai, a_c;
};

template <int D>
__device__ __forceinline__ CombineEntry combine_load(const AttnParams& p, int64_t e, int t, int64_t n_entries) {
  CombineEntry x;
  x.oo = -1;
  x.e = e;
  x.units = 0;
  x.fresh = false;
  x.li = x.l_c = 0.0f;
  x.ai = x.a_c = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (e >= n_entries) return x;
  const int h = (int)(e % p.hq);
  const int64_t vrow = e / p.hq;
  const int b = (int)(vrow / p.max_q);
  const int i = (int)(vrow - (int64_t)b * p.max_q);
  int nq = p.max_q, nk = p.max_k, qbase = 0;
  if (p.cu_q) {
    qbase = p.cu_q[b];
    nq = min(max(p.cu_q[b + 1] - qbase, 0), p.max_q);
  }
  if (p.cu_k) nk = p.cu_k[b + 1] - p.cu_k[b];
  if (i >= nq) return x;
  const int64_t orow = p.q_rows ? (int64_t)b * p.max_q + listed_row(p, b, qbase + i)
                                : (p.cu_q ? (int64_t)(qbase + i) : vrow);
  const int64_t oo = orow * p.hq + h;
  // (these loads go out before the decision is looked at: one round trip)
  // (A_in is read once: nontemporal.  The cached A_out is read again at
  // every step that reuses it, so it is loaded, and written by a recompute,
  // with ordinary accesses that let it stay in the caches between steps:
  // GQA long-context mean step 29.1-29.3 -> 28.7 us, LLaDA-like 10.13 ->
  // 9.93 us.)
  if (p.a_full) {
    x.li = p.l_cache[oo];
    x.ai = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p.a_cache + oo * D + 4 * t));
    if (p.decision) {
      x.l_c = p.l[oo];
      x.a_c = *reinterpret_cast<const f32x4*>(p.a + oo * D + 4 * t);
    }
  }
  x.units = p.kblocks ? p.n_kblocks : nk;
  // An empty prefix is written by the attention kernel's split 0.
  x.fresh = p.mode == kPrefixPartial && x.units > 0 && !(p.decision && p.decision[b * p.hq + h]);
  if (x.fresh || p.a_full) x.oo = oo;   // (else nothing to write)
  return x;
}

template <int D>
__device__ __forceinline__ void combine_finish(const AttnParams& p, const CombineEntry& x, int t,
                                               int64_t n_entries) {
  if (x.oo < 0) return;
  const int64_t oo = x.oo;
  f32x4 a_o;
  float l_o;
  if (x.fresh) {
    const int ns = (x.units + p.chunk - 1) / p.chunk;
    const float* la = p.ws_l + x.e;
    const float* aa = p.ws_a + x.e * D + 4 * t;
    const int64_t cs = n_entries;
    float mx = -INFINITY, den = 0.0f;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    constexpr int CB = 16;   // splits loaded per memory round trip
    for (int c0 = 0; c0 < ns; c0 += CB) {
      float lv[CB];
      f32x4 av[CB];
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        const bool ok = c0 + u < ns;
        lv[u] = ok ? la[(c0 + u) * cs] : -INFINITY;
        av[u] = ok ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(aa + (c0 + u) * cs * D))
                   : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
      float bm = mx;
#pragma unroll
      for (int u = 0; u < CB; ++u) bm = fmaxf(bm, lv[u]);
      const float r = __builtin_amdgcn_exp2f((mx - bm) * kLog2e);  // rescale earlier batches
      den *= r;
      acc *= r;
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        const float wgt = __builtin_amdgcn_exp2f((lv[u] - bm) * kLog2e);
        den += wgt;
        acc += wgt * av[u];
      }
      mx = bm;
    }
    a_o = acc * (1.0f / den);
    l_o = mx + __logf(den);
    *reinterpret_cast<f32x4*>(p.a + oo * D + 4 * t) = a_o;   // (the cache: kept cacheable, as above)
    if (t == 0) p.l[oo] = l_o;
  } else if (p.decision) {
    a_o = x.a_c;
    l_o = x.l_c;
  } else {
    a_o = *reinterpret_cast<const f32x4*>(p.a + oo * D + 4 * t);
    l_o = p.l[oo];
  }
  if (p.a_full) {
    // prefix part (cached or fresh) first, in-block part second
    const MergeWeights mw = merge_weights(l_o, x.li);
    f32x4 af;
#pragma unroll
    for (int k = 0; k < 4; ++k) af[k] = merge_elem(mw, a_o[k], x.ai[k]);
    __builtin_nontemporal_store(af, reinterpret_cast<f32x4*>(p.a_full + oo * D + 4 * t));
    if (t == 0 && p.l_full) p.l_full[oo] = mw.l;
  }
}

// N-way log-space merge of the split-KV partials (the merge equation applied
// across key splits), optionally followed by the merge with a precomputed
// in-block part.  D/4 threads per (row, head) entry, four dims each; a
// workgroup takes PER groups of 256/(D/4) consecutive entries (groups g and
// g + gridDim.x when PER == 2), whose first loads go out together.
//   p.mode == kPrefixPartial: entries whose prefix was recomputed combine the
//     split partials into A_out/L_out (p.a, p.l); the L and A partials of up
//     to 16 splits are loaded together, so one memory round trip serves a
//     batch.  Entries of reused heads (or of sequences with no prefix keys)
//     keep the A_out/L_out already in p.a/p.l.
//   p.mode == kPrefixFinal: A_out/L_out are already in p.a/p.l.
//   p.a_full != NULL: A_full/L_full = merge(A_out, L_out, A_in, L_in) with
//     A_in/L_in in p.a_cache/p.l_cache, for every entry.
template <int D, int PER>
__global__ void __launch_bounds__(256) combine_kernel(const AttnParams p) {
  constexpr int TPE = D / 4;
  constexpr int EPB = 256 / TPE;
  const int64_t n_entries = (int64_t)p.n_seq * p.max_q * p.hq;
  if (p.ready && blockIdx.x == 0)
    for (int c = 0; c < kReadyCopies; ++c)
      for (int b = threadIdx.x; b < p.n_seq; b += blockDim.x) p.ready[c * p.ready_stride + b] = 0;
  const int t = threadIdx.x % TPE;
  const int64_t e0 = (int64_t)blockIdx.x * EPB + threadIdx.x / TPE;
  if constexpr (PER == 1) {
    const CombineEntry x = combine_load<D>(p, e0, t, n_entries);
    combine_finish<D>(p, x, t, n_entries);
  } else {
    const int64_t e1 = e0 + (int64_t)gridDim.x * EPB;
    const CombineEntry x0 = combine_load<D>(p, e0, t, n_entries);
    const CombineEntry x1 = combine_load<D>(p, e1, t, n_entries);
    combine_finish<D>(p, x0, t, n_entries);
    combine_finish<D>(p, x1, t, n_entries);
  }
}

}  // namespace

hipError_t launch_combine(const AttnParams& p, int d, hipStream_t s) {
  const int64_t n_entries = (int64_t)p.n_seq * p.max_q * p.hq;
  const int64_t epb = 256 / (d / 4);
  const int64_t groups = (n_entries + epb - 1) / epb;
  // Large passes: two entry groups per workgroup (half the workgroups to
  // dispatch, two entries' loads in flight per thread); small ones keep one
  // group each, for more workgroups.
  const bool two = groups > 4 * (int64_t)device_cus();
  const dim3 grid((unsigned)(two ? (groups + 1) / 2 : groups));
  if (d == 128) {
    if (two) hipLaunchKernelGGL((combine_kernel<128, 2>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((combine_kernel<128, 1>), grid, dim3(256), 0, s, p);
  } else {
    if (two) hipLaunchKernelGGL((combine_kernel<64, 2>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((combine_kernel<64, 1>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

namespace {

// Groups (split, sequence, KV head) are dealt to the XCDs in turn, each with
// its row tiles on consecutive workgroups of its XCD (decode_item).
int item_grid(const AttnParams& p) { return item_grid_size(p); }


// p1 == nullptr: one part.  With two parts, p1's workgroups come first in
// the grid (dispatch order): the caller passes the in-block part as p1, so
// its real work starts at once while the prefix part's workgroups of reused
// heads exit.
template <int D, int RW, int KW, int KT, int ST, bool CAN_GATE = true>
hipError_t launch_variant(const AttnParams& p0, const AttnParams* p1, const GateParams* g, hipStream_t s) {
  const GateParams none{};
  const int g0 = item_grid(p0);
  if (!p1) {
    if (g0 == 0) return hipSuccess;
    hipLaunchKernelGGL((attn_bf16_kernel<D, RW, KW, KT, ST, false, false>), dim3(g0), dim3(64 * RW * KW), 0, s,
                       p0, p0, g0, none, 0);
    return hipGetLastError();
  }
  const int g1 = item_grid(*p1);
  if (g) {
    if constexpr (CAN_GATE) {
      const int gg = gate_grid(*g);
      hipLaunchKernelGGL((attn_bf16_kernel<D, RW, KW, KT, ST, true, true>), dim3(gg + g0 + g1),
                         dim3(64 * RW * KW), 0, s, *p1, p0, g1, *g, gg);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  if (g0 + g1 == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_bf16_kernel<D, RW, KW, KT, ST, true, false>), dim3(g0 + g1), dim3(64 * RW * KW), 0, s,
                     *p1, p0, g1, none, 0);
  return hipGetLastError();
}

template <int D, int NS>
hipError_t launch_pp(const AttnParams& p0, const AttnParams* p1, const GateParams* g, hipStream_t s) {
  const GateParams none{};
  const int g0 = item_grid(p0);
  if (!p1) {
    if (g0 == 0) return hipSuccess;
    hipLaunchKernelGGL((attn_pp_kernel<D, NS, false, false>), dim3(g0), dim3(512), 0, s, p0, p0, g0, none, 0);
    return hipGetLastError();
  }
  const int g1 = item_grid(*p1);
  if (g) {
    const int gg = gate_grid(*g);
    // A gated step under a count gate decides per sequence: its prefix part
    // runs as one persistent workgroup per compute unit (one fits per CU)
    // over the work items, reading their gate results in one batch.
    AttnParams pp = p0;
    int gp = g0;
    if (p0.decision != nullptr && p0.ready != nullptr && g->mode != BA_GATE_COSINE) {
      // (at most 64 items each: one pre-pass read per lane of a wave)
      pp.persist = std::min(g0, std::max(device_cus(), (g0 + 63) / 64));
      gp = pp.persist;
    }
    if (pp.persist > 0)
      hipLaunchKernelGGL((attn_pp_kernel<D, NS, true, true, true>), dim3(gg + gp + g1), dim3(512), 0, s, *p1, pp, g1,
                         *g, gg);
    else
      hipLaunchKernelGGL((attn_pp_kernel<D, NS, true, true>), dim3(gg + gp + g1), dim3(512), 0, s, *p1, pp, g1, *g,
                         gg);
    return hipGetLastError();
  }
  if (g0 + g1 == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_pp_kernel<D, NS, true, false>), dim3(g0 + g1), dim3(512), 0, s, *p1, p0, g1, none, 0);
  return hipGetLastError();
}

}  // namespace

// Variants (rows per workgroup x keys per iteration tile):
//   0: 128 rows (4 row-waves) x 64 keys, 2-stage ring (64 KB LDS at d=128:
//      2 WG per CU)
//   1:  64 rows (2 row-waves x 2 key-waves of 32) x 64 keys (2 WG per CU);
//       also used for fewer rows: the streaming, not the MFMA, sets the pace
//   2:  32 rows x 32 keys, one wave (32 KB LDS at d=128: 5 WG per CU): in-block
//       problems over short blocks, where latency dominates
//   3: 256 rows (two alternating groups of 4 waves) x 64 keys, 4-stage ring
//      (128 KB LDS at d=128: 1 WG per CU): many rows per KV head, where the
//      matrix cores set the pace
Bf16Plan plan_bf16(int d, int rows_per_kv_head, int max_k, bool prefix) {
  (void)d;
  // (an in-block problem with many keys is as MFMA-bound as a prefix pass)
  if (rows_per_kv_head > 192 && (prefix || max_k > 512)) return Bf16Plan{3, 256, 64, 1};
  // an in-block call over a short block is latency-bound whatever its row
  // count: one-wave workgroups of 32 rows give the most of them (the GQA
  // long-context in-block call, 256 rows per KV head over 64 keys: 12.6-12.9
  // -> 11.1-11.2 us against the 128-row workgroups)
  if (max_k <= 64 && !prefix) return Bf16Plan{2, 32, 32, 5};
  if (rows_per_kv_head > 64) return Bf16Plan{0, 128, 64, 2};
  return Bf16Plan{1, 64, 64, 2};
}

int max_splits_bf16(int d, int variant) {
  (void)d;
  (void)variant;
  return 256;
}

hipError_t launch_attn_bf16(const Bf16Plan& plan_in, const AttnParams& p, const AttnParams* p1, int d,
                            hipStream_t s, const GateParams* g_in) {
  if (g_in && !p1) return hipErrorInvalidValue;
  Bf16Plan plan = plan_in;
  // In the 256-row kernel every gate workgroup is as heavy as an attention
  // one (a whole CU's LDS), so the gates there use fewer, longer
  // workgroups: the count gates several positions per workgroup (about 128
  // workgroups in all; 64 and 256 were slower on the GQA long-context step),
  // the cosine gate fewer position chunks per (sequence, head) (about 128
  // workgroups; its workspace is sized for the most chunks).
  GateParams g_multi;
  const GateParams* g = g_in;
  if (g_in && plan.variant == 3) {
    g_multi = *g_in;
    if (g_in->mode != BA_GATE_COSINE) {
      const int64_t positions = (int64_t)g_in->n_blk * g_in->n_seq;
      int64_t ppw = (positions + 127) / 128;
      if (ppw < 1) ppw = 1;
      if (ppw > kMaxGatePositions) ppw = kMaxGatePositions;
      g_multi.pos_per_wg = (int)ppw;
    } else {
      const int64_t heads = (int64_t)g_in->hq * g_in->n_seq;
      int64_t ch = 128 / (heads > 0 ? heads : 1);
      if (ch < 1) ch = 1;
      if (ch < g_in->chunks) g_multi.chunks = (int)ch;
    }
    g = &g_multi;
  }
  // 32-key single-wave ring: in-block attention only
  if (plan.variant == 2 && (p.mode != kBlock || (p1 && p1->mode != kBlock))) plan.variant = 1;
  if (d == 128) {
    switch (plan.variant) {
      case 0: return launch_variant<128, 4, 1, 64, 2>(p, p1, g, s);
      case 1: return launch_variant<128, 2, 2, 32, 2>(p, p1, g, s);
      case 3: return launch_pp<128, 4>(p, p1, g, s);
      default: return launch_variant<128, 1, 1, 32, 2, false>(p, p1, g, s);
    }
  }
  switch (plan.variant) {
    case 0: return launch_variant<64, 4, 1, 64, 2>(p, p1, g, s);
    case 1: return launch_variant<64, 2, 2, 32, 2>(p, p1, g, s);
    case 3: return launch_pp<64, 4>(p, p1, g, s);
    default: return launch_variant<64, 1, 1, 32, 2, false>(p, p1, g, s);
  }
}

}  // namespace ba
