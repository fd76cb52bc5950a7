// bf16 matrix-core attention for gfx950: prefix (out-of-block) attention with
// split-KV, and in-block attention with the fused log-space merge.
//
// The computation is the split of FlashBlock (gist.science/es/paper/2602.05305,
// section 2, "Mecanismo Central"): each part yields an output A and its
// natural log-normaliser L = log Z; the parts are combined by the log-space
// merge equation of the same section.
//
// Per wave (64 lanes, 32 query rows):
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16, A = K tile (32 keys x 16 dims),
//                 B = Q^T (16 dims x 32 rows).  Lane l owns query row l%32;
//                 its 16 accumulator values per 32-key block are keys
//                 8j + 4(l/32) + i (j, i = 0..3).
//   softmax       online, in base 2 (scale*log2(e) folded into one FMA); the
//                 running row max is shared by the two lane halves through
//                 one v_permlane32_swap per tile; row sums stay per half and
//                 are added once at the end.
//   O^T += V^T P^T  A = V^T (32 dims x 16 keys) read from LDS, B = P^T taken
//                 straight from the S^T accumulators (8 consecutive
//                 accumulator values = one 16-key k-step), so P never leaves
//                 registers.
// Workgroup: RW row-waves x KW key-waves.  All waves stage the same K/V
// iteration tile (KW*KT keys) through LDS; key-wave kg processes keys
// [kg*KT, (kg+1)*KT) of it.  K is stored row-major (padded pitch), V is
// stored transposed [dim][key] with the key index's bits 2 and 3 swapped, so
// that each lane's eight PV operands are 16 contiguous bytes.  The next
// iteration tile is prefetched into registers while the current one is used.
// With KW > 1 the key-waves' partial results are merged through LDS by the
// same log-space rule.

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
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

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

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Position of key `kk` (index within one key-wave's tile) in the transposed V
// row: swap bits 2 and 3.
__device__ __forceinline__ int vt_pos(int kk) {
  return (kk & ~12) | ((kk & 4) << 1) | ((kk & 8) >> 1);
}

template <int D, int RW, int KW, int KT>
__global__ void __launch_bounds__(64 * RW * KW)
attn_bf16_kernel(const AttnParams p) {
  constexpr int NW = RW * KW;
  constexpr int NT = 64 * NW;
  constexpr int KTILE = KW * KT;                  // keys staged per iteration
  constexpr int KP = D * 2 + 16;                  // K row pitch, bytes
  constexpr int VP = KTILE * 2 + 16;              // V^T row pitch, bytes
  constexpr int KS = D / 16;                      // MFMA k-steps over head dim
  constexpr int DB = D / 32;                      // 32-dim output blocks
  constexpr int MB = KT / 32;                     // 32-key blocks per key-wave
  constexpr int CPR = D / 8;                      // 16-byte chunks per row
  constexpr int KTOT = KTILE * CPR;               // 16-byte K chunks per tile
  constexpr int VTOT = (KTILE / 4) * CPR;         // 4-key x 8-dim V blocks per tile
  constexpr int KCH = (KTOT + NT - 1) / NT;       // per thread
  constexpr int VCH = (VTOT + NT - 1) / NT;
  constexpr int SMEM_TILE = KTILE * KP + D * VP;
  constexpr int XSLOT = (DB * 16 + 2) * 64;       // floats per exchange slot
  constexpr int SMEM_X = (KW > 1) ? (KW - 1) * RW * XSLOT * 4 : 0;
  constexpr int SMEM = SMEM_TILE > SMEM_X ? SMEM_TILE : SMEM_X;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  unsigned char* const sK = smem;
  unsigned char* const sV = smem + KTILE * KP;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int rw = w % RW, kg = w / RW;
  const int lr = lane & 31, hf = lane >> 5;

  const int split = blockIdx.x, rt = blockIdx.y;
  const int b = blockIdx.z / p.hkv;
  const int kvh = blockIdx.z - b * p.hkv;
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
  if (p.mode == kPrefixPartial && kb >= nk) return;
  const int ke = min(nk, kb + p.chunk);
  const bool gated = p.decision != nullptr && p.mode != kBlock;
  if (gated) {
    const int rlast = min(R, row0 + RW * 32) - 1;
    bool any = false;
    for (int g = row0 / nq; g <= rlast / nq; ++g) any |= p.decision[b * p.hq + kvh * G + g] == 0;
    if (!any) return;
  }

  // This lane's query row.
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
    u32x4 x = rvalid ? ld16(qrow + 16 * ks + 8 * hf) : u32x4{0, 0, 0, 0};
    qf[ks] = __builtin_bit_cast(bf16x8, x);
  }

  const uint16_t* kptr = static_cast<const uint16_t*>(p.k) +
      (varlen ? (int64_t)kbase * p.ks1 : (int64_t)b * p.ks0) + (int64_t)kvh * p.ks2;
  const uint16_t* vptr = static_cast<const uint16_t*>(p.v) +
      (varlen ? (int64_t)kbase * p.vs1 : (int64_t)b * p.vs0) + (int64_t)kvh * p.vs2;

  u32x4 kreg[KCH];
  u32x4 vreg[VCH][4];
  auto load_tile = [&](int t0) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int c = tid + NT * u;
      const int key = c / CPR, col = c % CPR;
      const int j = (KTOT % NT == 0 || c < KTOT) ? t0 + key : ke;
      kreg[u] = (j < ke) ? ld16(kptr + (int64_t)j * p.ks1 + col * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < VCH; ++u) {
      const int c = tid + NT * u;
      const int kq = c / CPR, dg = c % CPR;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int j = (VTOT % NT == 0 || c < VTOT) ? t0 + 4 * kq + ii : ke;
        vreg[u][ii] = (j < ke) ? ld16(vptr + (int64_t)j * p.vs1 + dg * 8) : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int c = tid + NT * u;
      if (KTOT % NT != 0 && c >= KTOT) break;
      const int key = c / CPR, col = c % CPR;
      *reinterpret_cast<u32x4*>(sK + key * KP + col * 16) = kreg[u];
    }
#pragma unroll
    for (int u = 0; u < VCH; ++u) {
      const int c = tid + NT * u;
      if (VTOT % NT != 0 && c >= VTOT) break;
      const int kq = c / CPR, dg = c % CPR;
      const int key0 = 4 * kq;
      const int grp = key0 / KT;
      const int pos = grp * KT + vt_pos(key0 - grp * KT);
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const unsigned sel = (dd & 1) ? 0x07060302u : 0x05040100u;
        u32x2 pk;
        pk[0] = __builtin_amdgcn_perm(vreg[u][1][dd >> 1], vreg[u][0][dd >> 1], sel);
        pk[1] = __builtin_amdgcn_perm(vreg[u][3][dd >> 1], vreg[u][2][dd >> 1], sel);
        *reinterpret_cast<u32x2*>(sV + (dg * 8 + dd) * VP + pos * 2) = pk;
      }
    }
  };

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.0f;
  const float c2 = p.scale_log2;

  const int n_iter = (ke > kb) ? (ke - kb + KTILE - 1) / KTILE : 0;
  if (n_iter > 0) load_tile(kb);
  for (int it = 0; it < n_iter; ++it) {
    const int t0 = kb + it * KTILE;
    __syncthreads();
    store_tile();
    __syncthreads();
    if (it + 1 < n_iter) load_tile(t0 + KTILE);
    const int g0 = t0 + kg * KT;
    if (g0 >= ke) continue;

    f32x16 s[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      s[mb] = f32x16{};
      const unsigned char* krow = sK + (kg * KT + mb * 32 + lr) * KP + hf * 16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + ks * 32);
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
    mx = pair_max(mx);
    const float m_new = fmaxf(m_run, mx * c2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float ps = 0.0f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(s[mb][e], c2, -m_new));
        s[mb][e] = pv;
        ps += pv;
      }
    l_run = l_run * alpha + ps;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;

#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        u32x4 pw;
#pragma unroll
        for (int q = 0; q < 4; ++q) pw[q] = pack_bf16(s[mb][8 * h2 + 2 * q], s[mb][8 * h2 + 2 * q + 1]);
        const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
        const unsigned char* vcol = sV + (kg * KT + mb * 32 + 16 * h2 + 8 * hf) * 2;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vcol + (db * 32 + lr) * VP);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[db], 0, 0, 0);
        }
      }
    }
  }

  float l_tot = pair_sum(l_run);

  if constexpr (KW > 1) {
    __syncthreads();
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
    if (kg > 0) return;
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

  if (!rvalid) return;
  if (gated && p.decision[b * p.hq + h] != 0) return;

  const bool has = l_tot > 0.0f;
  const float inv = has ? 1.0f / l_tot : 0.0f;
  const float L = has ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  const int64_t orow = varlen ? (int64_t)(qbase + i) : (int64_t)b * p.max_q + i;
  const int64_t oe = orow * p.hq + h;

  if (p.mode != kBlock) {
    float* a;
    float* l;
    if (p.mode == kPrefixFinal) {
      a = p.a + oe * D;
      l = p.l + oe;
    } else {
      const int64_t ve = ((int64_t)split * p.n_seq * p.max_q + (int64_t)b * p.max_q + i) * p.hq + h;
      a = p.ws_a + ve * D;
      l = p.ws_l + ve;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 val = {o[db][4 * j] * inv, o[db][4 * j + 1] * inv, o[db][4 * j + 2] * inv,
                     o[db][4 * j + 3] * inv};
        *reinterpret_cast<f32x4*>(a + db * 32 + 8 * j + 4 * hf) = val;
      }
    if (hf == 0) *l = L;
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
    const float lc = p.l_cache[oe];
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
          const f32x4 cv = *reinterpret_cast<const f32x4*>(ac + c0);
          f32x4 val;
#pragma unroll
          for (int e = 0; e < 4; ++e) val[e] = fc * cv[e] + fi * o[db][4 * j + e];
          *reinterpret_cast<f32x4*>(af + c0) = val;
        }
    }
    if (p.l_full && hf == 0) p.l_full[oe] = lf;
  }
}

// N-way log-space merge of the split-KV partials of one (row, head) entry.
// D/4 threads per entry, 4 dims each.
__global__ void __launch_bounds__(256) combine_kernel(const CombineParams p) {
  const int tpe = p.d / 4;
  const int epb = blockDim.x / tpe;
  const int64_t e = (int64_t)blockIdx.x * epb + threadIdx.x / tpe;
  const int t = threadIdx.x % tpe;
  const int64_t n_entries = (int64_t)p.n_seq * p.max_q * p.hq;
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
  if (i >= nq) return;
  if (p.decision && p.decision[b * p.hq + h]) return;
  const int64_t orow = p.cu_q ? (int64_t)(qbase + i) : vrow;
  const int64_t oe = orow * p.hq + h;
  float* a = p.a + oe * p.d + 4 * t;
  const int ns = nk > 0 ? (nk + p.chunk - 1) / p.chunk : 0;
  if (ns == 0) {
    *reinterpret_cast<f32x4*>(a) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (t == 0) p.l[oe] = -INFINITY;
    return;
  }
  const int64_t sl = n_entries;  // entries per split
  float mx = -INFINITY;
  for (int c = 0; c < ns; ++c) mx = fmaxf(mx, p.ws_l[c * sl + e]);
  float den = 0.0f;
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int c = 0; c < ns; ++c) {
    const float wgt = __builtin_amdgcn_exp2f((p.ws_l[c * sl + e] - mx) * kLog2e);
    den += wgt;
    const f32x4 pa = *reinterpret_cast<const f32x4*>(p.ws_a + (c * sl + e) * p.d + 4 * t);
    acc += wgt * pa;
  }
  const float rd = 1.0f / den;
  *reinterpret_cast<f32x4*>(a) = acc * rd;
  if (t == 0) p.l[oe] = mx + __logf(den);
}

template <int D, int RW, int KW, int KT>
hipError_t launch_variant(const AttnParams& p, hipStream_t s) {
  dim3 grid(p.n_splits, p.row_tiles, p.n_seq * p.hkv);
  hipLaunchKernelGGL((attn_bf16_kernel<D, RW, KW, KT>), grid, dim3(64 * RW * KW), 0, s, p);
  return hipGetLastError();
}

}  // namespace

// Variants: 0 = 128 rows x 64 keys (4 row-waves), 1 = 64 rows x 2x32 keys,
// 2 = 32 rows x 4x32 keys.  Fewer query rows per KV head -> more key-waves,
// so a workgroup still keeps four waves busy.
Bf16Plan plan_bf16(int d, int rows_per_kv_head, int max_k, bool prefix) {
  (void)d;
  (void)max_k;
  (void)prefix;
  if (rows_per_kv_head > 64) return Bf16Plan{0, 128, 64};
  if (rows_per_kv_head > 32) return Bf16Plan{1, 64, 64};
  return Bf16Plan{2, 32, 128};
}

hipError_t launch_attn_bf16(const Bf16Plan& plan, const AttnParams& p, int d, hipStream_t s) {
  if (d == 128) {
    switch (plan.variant) {
      case 0: return launch_variant<128, 4, 1, 64>(p, s);
      case 1: return launch_variant<128, 2, 2, 32>(p, s);
      default: return launch_variant<128, 1, 4, 32>(p, s);
    }
  }
  switch (plan.variant) {
    case 0: return launch_variant<64, 4, 1, 64>(p, s);
    case 1: return launch_variant<64, 2, 2, 32>(p, s);
    default: return launch_variant<64, 1, 4, 32>(p, s);
  }
}

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
  const int tpe = p.d / 4;
  const int epb = 256 / tpe;
  const int64_t n = (int64_t)p.n_seq * p.max_q * p.hq;
  const int64_t blocks = (n + epb - 1) / epb;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace ba
