// Internal interfaces between the C-ABI front end (ba_api.hip) and the
// kernel translation units.  Nothing here is exported.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

#include "ba.h"

namespace ba {

// What an attention launch writes.
enum AttnMode : int {
  kPrefixFinal = 0,   // prefix attention, one split: A_out/L_out directly
  kPrefixPartial = 1, // prefix attention, split k: partials into the workspace
  kBlock = 2,         // in-block attention (+ optional fused merge)
};

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  int64_t qs0, qs1, qs2;
  int64_t ks0, ks1, ks2;
  int64_t vs0, vs1, vs2;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const uint8_t* decision;
  int n_seq, hq, hkv, group, max_q, max_k;
  float scale_log2;   // softmax scale * log2(e)
  int chunk;          // keys per split
  int n_splits;
  int row_tiles;      // row tiles per (sequence, KV head)
  int mode;
  // outputs / merge inputs
  float* a;           // A_out (prefix final) or A_in (block), may be null in block mode
  float* l;
  float* ws_a;        // [n_splits][n_seq*max_q][hq][d]
  float* ws_l;        // [n_splits][n_seq*max_q][hq]
  const float* a_cache;
  const float* l_cache;
  float* a_full;
  float* l_full;
  // Gate run by the same launch: a gated prefix part first waits until the
  // gate has published sequence b's result in ready[b] (count mode: M_b,
  // from which it decides itself against gate_tau; cosine mode: all hq
  // decisions written), polling copy (workgroup % kReadyCopies) of the
  // ready words at most spin_limit times; a wait that gives up counts itself
  // in *gave_up (if set) and computes its heads into the split workspace
  // (mode kPrefixPartial), where the combine pass applies the decisions.
  // The combine pass after such a launch zeroes ready[0 .. n_seq) of every
  // copy.
  int32_t* ready;
  int ready_stride;
  int spin_limit;
  int32_t* gave_up;
  // > 0: the gated prefix part of a count-gated fused launch runs as this
  // many persistent workgroups, workgroup i taking work items i, i + persist,
  // ... of the part's grid and computing only those whose sequence
  // recomputes.
  int persist;
  int gate_mode;
  int gate_tau;
  // Key-block list mode (dense prefix only): (sequence, KV head) attends over
  // the keys of blocks kblocks[(b*hkv + kvh)*n_kblocks + i], i < n_kblocks,
  // block j being keys [kBlockKeys*j, kBlockKeys*(j+1)) clipped to max_k;
  // chunk and the item key ranges then count list entries, not keys.
  const int32_t* kblocks;
  int n_kblocks;
  // Row-list mode (dense prefix only, with cu_q set and cu_k NULL): the
  // query rows of sequence b are list entries j in [cu_q[b], cu_q[b+1]),
  // entry j naming the dense row q_rows[j] = b * max_q + position; Q is read
  // and A_out/L_out written at that dense row, other rows stay untouched.
  const int32_t* q_rows;
};
constexpr int kBlockKeys = 64;   // keys per listed key block = the prefix kernels' tile

// Row-list mode: the position named by list entry j of sequence b, clamped
// into [0, max_q) so that bad device data can give a wrong result but never
// an access outside Q or the cache.
__device__ __forceinline__ int listed_row(const AttnParams& p, int b, int j) {
  const int pos = p.q_rows[j] - b * p.max_q;
  return min(max(pos, 0), p.max_q - 1);
}


// Launch-shape choice for the bf16 matrix-core kernel.
struct Bf16Plan {
  int variant;        // index into the instantiated kernel table
  int rows_per_wg;    // query rows one workgroup covers
  int keys_per_iter;  // keys one workgroup stages per iteration
  int wg_per_cu;      // workgroups that fit on one compute unit (LDS bound)
};

Bf16Plan plan_bf16(int d, int rows_per_kv_head, int max_k, bool prefix);
int max_splits_bf16(int d, int variant);
hipError_t launch_attn_f32(const AttnParams& p, int d, hipStream_t s);
// After a prefix launch: combines split partials (p.mode == kPrefixPartial)
// into p.a/p.l and, if p.a_full is set, merges A_out/L_out with A_in/L_in
// (p.a_cache/p.l_cache) into p.a_full/p.l_full for every (row, head).
hipError_t launch_combine(const AttnParams& p, int d, hipStream_t s);

struct MergeParams {
  int64_t rows;
  int d;
  const float* a1;
  const float* l1;
  const float* a2;
  const float* l2;
  float* a;
  float* l;
};
hipError_t launch_merge(const MergeParams& p, hipStream_t s);

struct GateParams {
  int mode, esize;
  int n_seq, n_blk, hq, hkv, d;
  const void* q_cur;
  const void* q_prev;
  int64_t qs0, qs1, qs2;
  const void* k_cur;
  const void* k_prev;
  const void* v_cur;
  const void* v_prev;
  int64_t ks0, ks1, ks2;
  const uint8_t* upd_mask;
  int tau;
  double gamma;
  int cache_valid;
  int chunks;          // cosine mode: position chunks per (sequence, head)
  int vec16;           // 1 if every row start is 16-byte aligned
  int32_t* m_count;
  double* cos;
  uint8_t* decision;
  int32_t* ws_int;     // tickets / counters
  double* ws_dbl;      // cosine partials
  int32_t* ready;      // NULL, or the ready words (kReadyCopies copies)
  int ready_stride;    // ints between copies
  uint8_t* since;      // cumulative count mode: positions updated since the last refresh
  int pos_per_wg;      // count modes: block positions per workgroup (1 .. 32)
  // fused step only: the waiting prefix workgroups' poll bound and give-up count
  int spin_limit;
  int32_t* gave_up;
};
constexpr int kReadyCopies = 4;
constexpr int kMaxGatePositions = 32;   // count-gate positions per workgroup (one mask bit each)
int gate_grid(const GateParams& p);

// One launch; with p1 non-NULL it also runs the independent part p1 (same
// variant; its row tiles counted for plan.rows_per_wg).  With g non-NULL as
// well, the gate runs in the first workgroups of the same launch and the
// prefix part p waits for it per sequence (p.ready == g->ready).
hipError_t launch_attn_bf16(const Bf16Plan& plan, const AttnParams& p, const AttnParams* p1, int d,
                            hipStream_t s, const GateParams* g = nullptr);
int gate_cos_chunks(int n_blk, int d);
size_t gate_workspace_bytes(int mode, int n_seq, int hq, int n_blk, int d);
hipError_t launch_gate(const GateParams& p, hipStream_t s);

// KL lock criterion: one row per token, both steps' logits over the vocabulary.
struct KlParams {
  int n;                  // token rows
  int64_t vocab;
  int64_t stride;         // elements between rows
  int esize;              // 2 (bf16) or 4 (float32)
  int vec;                // 1 if rows start 16-byte aligned (vector loads)
  const void* cur;
  const void* prev;
  const uint8_t* eligible;
  float eps;
  float* kl;
  uint8_t* locked;
};
hipError_t launch_kl_lock(const KlParams& p, hipStream_t s);

constexpr int kMaxBranches = 512;
struct PackParams {
  int n_branch;
  int n_total;
  const uint8_t* locked;
  int32_t* cu;
  int32_t* gather;
  int32_t* total;
  int esize, h, d;
  const void* q_src;
  int64_t qs0, qs1;
  void* q_packed;
  int vec16;   // 1 if every copied row start is 16-byte aligned
};
hipError_t launch_pack(const PackParams& p, const int32_t* starts_host, hipStream_t s);

}  // namespace ba
