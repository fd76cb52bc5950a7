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
// (no register round trip) into an ST-deep ring of stages; a tile is waited
// for with s_waitcnt vmcnt and one barrier per iteration, so ST-1 tiles are
// in flight while one is consumed.  Rows of K and V are 2*d bytes; their
// 16-byte chunks are XOR-swizzled by row so that both the 32-row K reads
// (ds_read_b128) and the 4-row V transpose reads hit distinct banks.
// Workgroup: RW row-waves x KW key-waves; key-wave kg takes keys
// [kg*KT, (kg+1)*KT) of each KW*KT-key iteration tile, and the key-waves'
// partial results are merged through LDS at the end.
// Work mapping: work items are numbered so that the row tiles and key splits
// sharing one (sequence, KV head) are consecutive, and consecutive items go
// to the same XCD (workgroup i runs on XCD i % 8), so K/V re-reads hit that
// XCD's L2.

#include <math.h>

#include "ba_internal.h"

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

__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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

// Wait until at most N vector-memory operations of this wave are in flight,
// then barrier the workgroup.  The memory clobber keeps the compiler from
// moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int D>
__device__ __forceinline__ int swz(int row) {
  return D == 128 ? ((row & 7) << 1) : ((row & 3) << 1);
}

template <int D, int RW, int KW, int KT, int ST, bool GATED>
__global__ void __launch_bounds__(64 * RW * KW)
    __attribute__((amdgpu_waves_per_eu(ST * 4 * KW * KT * D > 80 * 1024 ? 1 : 2)))
attn_bf16_kernel(const AttnParams p) {
  constexpr int NW = RW * KW;
  constexpr int KTILE = KW * KT;                 // keys per iteration tile
  constexpr int ROWB = D * 2;                    // bytes per K/V row
  constexpr int CPR = D / 8;                     // 16-byte chunks per row
  constexpr int RPB = 1024 / ROWB;               // rows per 1 KB DMA block
  constexpr int TILE_B = KTILE * ROWB;           // bytes of one K (or V) tile
  constexpr int NBLK = TILE_B / 1024;            // DMA blocks per K (or V) tile
  constexpr int BPW = NBLK / NW;                 // DMA blocks per wave
  constexpr int LPT = 2 * BPW;                   // DMA ops per thread per tile
  constexpr int KS = D / 16;                     // MFMA k-steps over head dim
  constexpr int DB = D / 32;                     // 32-dim output blocks
  constexpr int MB = KT / 32;                    // 32-key blocks per key-wave
  static_assert(NBLK % NW == 0 && BPW >= 1, "tile must split evenly into per-wave DMA blocks");
  static_assert(ST >= 2 && ST <= 4, "ring depth");
  constexpr int STAGE_B = 2 * TILE_B;
  constexpr int XSLOT = (DB * 16 + 2) * 64;      // floats per key-wave exchange slot
  constexpr int SMEM_X = (KW > 1) ? (KW - 1) * RW * XSLOT * 4 : 0;
  constexpr int SMEM_R = ST * STAGE_B;
  constexpr int SMEM = SMEM_R > SMEM_X ? SMEM_R : SMEM_X;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[SMEM];
  const unsigned smem_base = (unsigned)(uintptr_t)smem;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int rw = w % RW, kg = w / RW;
  const int lr = lane & 31, hf = lane >> 5;

  // --- work item (XCD-aware numbering) ---
  const int n_items = p.n_splits * p.row_tiles * p.n_seq * p.hkv;
  const int per_xcd = (n_items + kXcds - 1) / kXcds;
  const int item = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (item >= n_items) return;
  const int split = item % p.n_splits;
  const int rt = (item / p.n_splits) % p.row_tiles;
  const int bz = item / (p.n_splits * p.row_tiles);
  const int b = bz / p.hkv;
  const int kvh = bz - b * p.hkv;

  const bool varlen = p.cu_q != nullptr;
  int qbase = 0, nq = p.max_q, kbase = 0, nk = p.max_k;
  if (varlen) {
    qbase = p.cu_q[b];
    nq = p.cu_q[b + 1] - qbase;
    kbase = p.cu_k[b];
    nk = p.cu_k[b + 1] - kbase;
  }
  const int G = p.group;
  const int R = G * nq;
  const int row0 = rt * (RW * 32);
  if (row0 >= R) return;
  const int kb = split * p.chunk;
  // A sequence with no keys at all is finished by split 0 alone (A = 0,
  // L = -inf); otherwise splits past the end have nothing to do.
  const int mode = (p.mode == kPrefixPartial && nk == 0) ? kPrefixFinal : p.mode;
  if (p.mode == kPrefixPartial && kb >= nk && !(nk == 0 && split == 0)) return;
  const int ke = min(nk, kb + p.chunk);
  if constexpr (GATED) {
    const int rlast = min(R, row0 + RW * 32) - 1;
    bool any = false;
    for (int g = row0 / nq; g <= rlast / nq; ++g) any |= p.decision[b * p.hq + kvh * G + g] == 0;
    if (!any) return;
  }

  // --- this lane's query row and its Q operand (B of S^T = K Q^T) ---
  const int r = row0 + rw * 32 + lr;
  const bool rvalid = r < R;
  const int g = rvalid ? r / nq : 0;
  const int i = rvalid ? r - g * nq : 0;
  const int h = kvh * G + g;
  const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
      (varlen ? (int64_t)(qbase + i) * p.qs1 : (int64_t)b * p.qs0 + (int64_t)i * p.qs1) +
      (int64_t)h * p.qs2;
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 x = rvalid ? *reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * hf) : u32x4{0, 0, 0, 0};
    qf[ks] = __builtin_bit_cast(bf16x8, x);
  }

  const uint16_t* kptr = static_cast<const uint16_t*>(p.k) +
      (varlen ? (int64_t)kbase * p.ks1 : (int64_t)b * p.ks0) + (int64_t)kvh * p.ks2;
  const uint16_t* vptr = static_cast<const uint16_t*>(p.v) +
      (varlen ? (int64_t)kbase * p.vs1 : (int64_t)b * p.vs0) + (int64_t)kvh * p.vs2;

  // DMA of one iteration tile (keys t0 .. t0+KTILE) into ring stage st.
  // Lane l of a 1 KB block writes row blk*RPB + l/CPR, chunk slot l%CPR, which
  // holds source chunk (l%CPR) ^ swz(row).  Keys past the range are clamped
  // to the last valid key (finite data; their scores are masked).
  const int l_row = lane / CPR;
  const int l_slot = lane % CPR;
  auto issue_tile = [&](int t0, int st) {
    const unsigned kdst = smem_base + st * STAGE_B;
    const unsigned vdst = kdst + TILE_B;
#pragma unroll
    for (int u = 0; u < BPW; ++u) {
      const int blk = w * BPW + u;
      const int row = blk * RPB + l_row;
      const int c = l_slot ^ swz<D>(row);
      const int j = min(t0 + row, ke - 1);
      dma16(kptr + (int64_t)j * p.ks1 + c * 8, kdst + blk * 1024);
      dma16(vptr + (int64_t)j * p.vs1 + c * 8, vdst + blk * 1024);
    }
  };

  // Single-wave workgroups serve small in-block problems, where the cache read
  // of the merge would otherwise be one more memory round trip after the
  // compute: fetch this lane's cached A_out/L_out now.
  constexpr bool kPrefetchCache = (NW == 1);
  f32x4 cache_a[kPrefetchCache ? 4 * DB : 1];
  float cache_l = 0.0f;
  if constexpr (kPrefetchCache) {
    if (p.mode == kBlock && p.a_cache && rvalid) {
      const int64_t ce = (varlen ? (int64_t)(qbase + i) : (int64_t)b * p.max_q + i) * p.hq + h;
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

  // V operand lanes: 16-lane group tq covers dims db*32 + (tq%2)*16 .. +15;
  // source lane ts addresses key row k0 + ts/4, dims +4*(ts%4) .. +3, i.e.
  // chunk 4db + 2(tq%2) + (ts%4)/2, half ts%2.
  const int tq = lane >> 4, ts = lane & 15;

  const int n_iter = (ke > kb) ? (ke - kb + KTILE - 1) / KTILE : 0;
#pragma unroll
  for (int s = 0; s < ST - 1; ++s)
    if (s < n_iter) issue_tile(kb + s * KTILE, s);

  for (int it = 0; it < n_iter; ++it) {
    const int ahead = min(ST - 2, n_iter - 1 - it);   // tiles issued after this one
    if constexpr (ST == 2) {
      wait_barrier<0>();
    } else if constexpr (ST == 3) {
      if (ahead >= 1) wait_barrier<LPT>(); else wait_barrier<0>();
    } else {
      if (ahead >= 2) wait_barrier<2 * LPT>();
      else if (ahead == 1) wait_barrier<LPT>();
      else wait_barrier<0>();
    }
    if (it + ST - 1 < n_iter) issue_tile(kb + (it + ST - 1) * KTILE, (it + ST - 1) % ST);

    const int t0 = kb + it * KTILE;
    const int g0 = t0 + kg * KT;
    if (g0 >= ke) continue;
    const unsigned char* sK = smem + (it % ST) * STAGE_B;
    const unsigned char* sV = sK + TILE_B;

    f32x16 s[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      s[mb] = f32x16{};
      const int row = kg * KT + mb * 32 + lr;
      const unsigned char* krow = sK + row * ROWB;
      const int sw = swz<D>(row);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + (((2 * ks + hf) ^ sw) << 4));
        s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[mb], 0, 0, 0);
      }
    }
    if (g0 + KT > ke) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = g0 + mb * 32 + 8 * (e >> 2) + 4 * hf + (e & 3);
          if (key >= ke) s[mb][e] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[mb][e]);
    mx = pair_max(mx) * c2;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
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
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        u32x4 pw;
#pragma unroll
        for (int q = 0; q < 4; ++q) pw[q] = pack_bf16(s[mb][8 * h2 + 2 * q], s[mb][8 * h2 + 2 * q + 1]);
        const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
        const int kbase16 = kg * KT + mb * 32 + 16 * h2;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int c = 4 * db + 2 * (tq & 1) + ((ts & 3) >> 1);
          i16x4 lo, hi;
          {
            const int row = kbase16 + 4 * hf + (ts >> 2);
            const unsigned char* a = sV + row * ROWB + ((c ^ swz<D>(row)) << 4) + 8 * (ts & 1);
            lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(a));
          }
          {
            const int row = kbase16 + 8 + 4 * hf + (ts >> 2);
            const unsigned char* a = sV + row * ROWB + ((c ^ swz<D>(row)) << 4) + 8 * (ts & 1);
            hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(a));
          }
          const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[db], 0, 0, 0);
        }
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
  if constexpr (GATED) writer = writer && p.decision[b * p.hq + h] == 0;
  const bool has = l_tot > 0.0f;
  const float inv = has ? 1.0f / l_tot : 0.0f;
  const float L = has ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  const int64_t orow = varlen ? (int64_t)(qbase + i) : (int64_t)b * p.max_q + i;
  const int64_t oe = orow * p.hq + h;

  if (mode == kPrefixPartial) {
    // This split's partial result (normalised A and its L); the combine
    // kernel merges the splits.
    if (writer) {
      const int64_t n_entries = (int64_t)p.n_seq * p.max_q * p.hq;
      const int64_t ve = (int64_t)split * n_entries + ((int64_t)b * p.max_q + i) * p.hq + h;
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
    if constexpr (kPrefetchCache) lc = cache_l; else lc = p.l_cache[oe];
    const float mm = fmaxf(lc, L);
    float wc = 0.0f, wi = 0.0f, lf = -INFINITY, rden = 0.0f;
    if (mm != -INFINITY) {
      wc = __builtin_amdgcn_exp2f((lc - mm) * kLog2e);
      wi = __builtin_amdgcn_exp2f((L - mm) * kLog2e);
      const float den = wc + wi;
      rden = 1.0f / den;
      lf = mm + __logf(den);
    }
    const float fc = wc * rden, fi = wi * rden * inv;
    if (p.a_full) {
      const float* ac = p.a_cache + oe * D;
      float* af = p.a_full + oe * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c0 = db * 32 + 8 * j + 4 * hf;
          f32x4 cv;
          if constexpr (kPrefetchCache) cv = cache_a[db * 4 + j]; else cv = *reinterpret_cast<const f32x4*>(ac + c0);
          f32x4 val;
#pragma unroll
          for (int e = 0; e < 4; ++e) val[e] = fc * cv[e] + fi * o[db][4 * j + e];
          *reinterpret_cast<f32x4*>(af + c0) = val;
        }
    }
    if (p.l_full && hf == 0) p.l_full[oe] = lf;
  }
}


// N-way log-space merge of the split-KV partials (the merge equation applied
// across key splits).  D/4 threads per (row, head) entry, four dims each; the
// L and A partials of up to 8 splits are loaded together, so one memory
// round trip serves a batch.
template <int D>
__global__ void __launch_bounds__(256) combine_kernel(const AttnParams p) {
  constexpr int TPE = D / 4;
  constexpr int EPB = 256 / TPE;
  const int64_t n_entries = (int64_t)p.n_seq * p.max_q * p.hq;
  const int64_t e = (int64_t)blockIdx.x * EPB + threadIdx.x / TPE;
  const int t = threadIdx.x % TPE;
  if (e >= n_entries) return;
  const int h = (int)(e % p.hq);
  const int64_t vrow = e / p.hq;
  const int b = (int)(vrow / p.max_q);
  const int i = (int)(vrow - (int64_t)b * p.max_q);
  int nq = p.max_q, nk = p.max_k, qbase = 0;
  if (p.cu_q) {
    qbase = p.cu_q[b];
    nq = p.cu_q[b + 1] - qbase;
    nk = p.cu_k[b + 1] - p.cu_k[b];
  }
  if (i >= nq || nk == 0) return;  // empty prefix: written by the attention kernel
  if (p.decision && p.decision[b * p.hq + h]) return;
  const int ns = (nk + p.chunk - 1) / p.chunk;
  const float* la = p.ws_l + e;
  const float* aa = p.ws_a + e * D + 4 * t;
  const int64_t cs = n_entries;
  float mx = -INFINITY, den = 0.0f;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int c0 = 0; c0 < ns; c0 += 8) {
    float lv[8];
    f32x4 av[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool ok = c0 + u < ns;
      lv[u] = ok ? la[(c0 + u) * cs] : -INFINITY;
      av[u] = ok ? *reinterpret_cast<const f32x4*>(aa + (c0 + u) * cs * D) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    float bm = mx;
#pragma unroll
    for (int u = 0; u < 8; ++u) bm = fmaxf(bm, lv[u]);
    const float r = __builtin_amdgcn_exp2f((mx - bm) * kLog2e);  // rescale earlier batches
    den *= r;
    acc *= r;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float wgt = __builtin_amdgcn_exp2f((lv[u] - bm) * kLog2e);
      den += wgt;
      acc += wgt * av[u];
    }
    mx = bm;
  }
  const int64_t oo = (p.cu_q ? (int64_t)(qbase + i) : vrow) * p.hq + h;
  *reinterpret_cast<f32x4*>(p.a + oo * D + 4 * t) = acc * (1.0f / den);
  if (t == 0) p.l[oo] = mx + __logf(den);
}

template <int D, int RW, int KW, int KT, int ST>
hipError_t launch_variant(const AttnParams& p, hipStream_t s) {
  const int n_items = p.n_splits * p.row_tiles * p.n_seq * p.hkv;
  const int per_xcd = (n_items + kXcds - 1) / kXcds;
  dim3 grid(per_xcd * kXcds);
  if (p.decision != nullptr && p.mode != kBlock)
    hipLaunchKernelGGL((attn_bf16_kernel<D, RW, KW, KT, ST, true>), grid, dim3(64 * RW * KW), 0, s, p);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<D, RW, KW, KT, ST, false>), grid, dim3(64 * RW * KW), 0, s, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || p.mode != kPrefixPartial) return err;
  const int64_t n_entries = (int64_t)p.n_seq * p.max_q * p.hq;
  const int64_t epb = 256 / (D / 4);
  hipLaunchKernelGGL((combine_kernel<D>), dim3((unsigned)((n_entries + epb - 1) / epb)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

// Variants (rows per workgroup x keys per iteration tile, 2-stage ring):
//   0: 128 rows (4 row-waves) x 64 keys (64 KB LDS at d=128: 2 WG per CU)
//   1:  64 rows (2 row-waves x 2 key-waves of 32) x 64 keys (2 WG per CU);
//       also used for fewer rows: the streaming, not the MFMA, sets the pace
//   2:  32 rows x 32 keys, one wave (8 KB LDS at d=128): small in-block
//       problems, where latency dominates
Bf16Plan plan_bf16(int d, int rows_per_kv_head, int max_k, bool prefix) {
  (void)d;
  if (rows_per_kv_head > 64) return Bf16Plan{0, 128, 64, 2};
  if (rows_per_kv_head <= 32 && max_k <= 64 && !prefix) return Bf16Plan{2, 32, 32, 8};
  return Bf16Plan{1, 64, 64, 2};
}

int max_splits_bf16(int d, int variant) {
  (void)d;
  (void)variant;
  return 256;
}

hipError_t launch_attn_bf16(const Bf16Plan& plan, const AttnParams& p, int d, hipStream_t s) {
  if (d == 128) {
    switch (plan.variant) {
      case 0: return launch_variant<128, 4, 1, 64, 2>(p, s);
      case 1: return launch_variant<128, 2, 2, 32, 2>(p, s);
      default: return launch_variant<128, 1, 1, 32, 2>(p, s);
    }
  }
  switch (plan.variant) {
    case 0: return launch_variant<64, 4, 1, 64, 2>(p, s);
    case 1: return launch_variant<64, 2, 2, 32, 2>(p, s);
    default: return launch_variant<64, 1, 1, 32, 2>(p, s);
  }
}

}  // namespace ba
