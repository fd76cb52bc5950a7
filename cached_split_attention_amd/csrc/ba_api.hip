// C-ABI front end: argument validation, launch planning and dispatch.
// Every check happens before the first launch, so a non-OK status means
// nothing was enqueued.

#include <math.h>

#include <cmath>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "ba_internal.h"

namespace {

thread_local std::string g_err;

// Default polls (each an agent-scope load and a short sleep, about a
// microsecond) a prefix workgroup makes for the gate of its own launch before
// it gives up and computes its heads into the split workspace; far above the
// gate's running time.  The gate descriptor's wait_polls overrides it.
constexpr int kGateSpinLimit = 1 << 20;

ba_status fail(ba_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

ba_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return BA_OK;
  return fail(BA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int esize_of(int dtype) { return dtype == BA_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Resolved shape of one attention request.
struct AttnShape {
  int group;
  bool varlen;
  float scale;
};

ba_status check_desc(const ba_attn_desc* d, AttnShape* out) {
  if (!d) return fail(BA_ERR_NULL, "descriptor is NULL");
  if (d->dtype != BA_BF16 && d->dtype != BA_F32) return fail(BA_ERR_DTYPE, "unknown dtype %d", d->dtype);
  if (d->n_seq < 0 || d->max_q < 0 || d->max_k < 0)
    return fail(BA_ERR_SHAPE, "negative size (n_seq %d, max_q %d, max_k %d)", d->n_seq, d->max_q, d->max_k);
  if (d->hq < 1 || d->hkv < 1) return fail(BA_ERR_SHAPE, "hq %d and hkv %d must be >= 1", d->hq, d->hkv);
  if (d->hq % d->hkv) return fail(BA_ERR_SHAPE, "hq %d is not a multiple of hkv %d", d->hq, d->hkv);
  if (d->d != 64 && d->d != 128) return fail(BA_ERR_UNSUPPORTED, "head dim %d (supported: 64, 128)", d->d);
  if ((d->cu_q == nullptr) != (d->cu_k == nullptr))
    return fail(BA_ERR_SHAPE, "cu_q and cu_k must both be set (varlen) or both be NULL (dense)");
  const bool varlen = d->cu_q != nullptr;
  const bool has_rows = d->n_seq > 0 && d->max_q > 0;
  if (has_rows && !d->q) return fail(BA_ERR_NULL, "q is NULL");
  if (has_rows && d->max_k > 0 && (!d->k || !d->v)) return fail(BA_ERR_NULL, "k or v is NULL");
  const int64_t* st[3] = {d->q_stride, d->k_stride, d->v_stride};
  const char* nm[3] = {"q", "k", "v"};
  const int es = esize_of(d->dtype);
  for (int t = 0; t < 3; ++t) {
    for (int a = 0; a < 3; ++a)
      if (st[t][a] < 0) return fail(BA_ERR_SHAPE, "%s_stride[%d] = %lld is negative", nm[t], a, (long long)st[t][a]);
    for (int a = varlen ? 1 : 0; a < 3; ++a)
      if ((st[t][a] * es) % 16)
        return fail(BA_ERR_UNSUPPORTED, "%s_stride[%d] = %lld elements is not a multiple of 16 bytes", nm[t], a,
                    (long long)st[t][a]);
  }
  if ((d->q && !aligned16(d->q)) || (d->k && !aligned16(d->k)) || (d->v && !aligned16(d->v)))
    return fail(BA_ERR_UNSUPPORTED, "q, k and v must be 16-byte aligned");
  if ((int64_t)d->n_seq * d->hkv > 65535 && !varlen)
    return fail(BA_ERR_UNSUPPORTED, "n_seq * hkv = %lld exceeds 65535", (long long)d->n_seq * d->hkv);
  if ((int64_t)d->n_seq * d->hkv > 65535) return fail(BA_ERR_UNSUPPORTED, "n_seq * hkv exceeds 65535");
  // (rows per KV head, hq / hkv * max_q, are numbered with 32-bit integers)
  if ((int64_t)(d->hq / d->hkv) * d->max_q > (1LL << 30))
    return fail(BA_ERR_UNSUPPORTED, "hq / hkv * max_q = %lld rows per KV head exceeds 2^30",
                (long long)(d->hq / d->hkv) * d->max_q);
  out->group = d->hq / d->hkv;
  out->varlen = varlen;
  out->scale = d->scale > 0.0f ? d->scale : 1.0f / sqrtf((float)d->d);
  return BA_OK;
}

// Split-KV plan for prefix attention.
struct PrefixPlan {
  ba::Bf16Plan bf;
  int row_tiles;
  int n_splits;
  int chunk;
};

// n_kblocks >= 0: key-block list mode, one iteration tile per listed block
// and at most 64 list entries per workgroup; chunk then counts entries.
// shares >= 1: the call is gated (valid cache), so an unknown share of the
// work items recomputes; the makespan estimate is then averaged over shares
// k/shares, k = 1 .. shares, weighted 1/k (a gate makes small recomputed
// subsets the common case; smaller splits keep a step that recomputes few
// heads or sequences short), and over the step that recomputes nothing,
// weighted 1, whose workgroups only read their decision and leave (about
// half a tile each, per round of slots).  shares == 0: ungated, the full
// share only.
// per_seq: the gate decides per sequence (count gates).  With the 256-row
// kernel such a gated step runs its prefix part as persistent workgroups
// (one per compute unit) that read their items' gate results in one batch:
// a step that reuses everything then costs about one round of reads
// whatever the split, and the combine pass only handles the recomputing
// share's partials, so both terms are modelled that way.
PrefixPlan plan_prefix(const ba_attn_desc* d, int group, int n_kblocks = -1, int shares = 0, bool per_seq = false) {
  PrefixPlan pp{};
  if (d->dtype == BA_F32) {
    pp.row_tiles = 1;
    pp.n_splits = 1;
    pp.chunk = d->max_k > 0 ? d->max_k : 1;
    return pp;
  }
  const int rows = group * d->max_q;
  pp.bf = ba::plan_bf16(d->d, rows, d->max_k, true);
  pp.row_tiles = (rows + pp.bf.rows_per_wg - 1) / pp.bf.rows_per_wg;
  if (pp.row_tiles < 1) pp.row_tiles = 1;
  const int64_t items = (int64_t)d->n_seq * d->hkv * pp.row_tiles;
  const int kpi = pp.bf.keys_per_iter;
  const bool listed = n_kblocks >= 0;
  const int64_t iters = listed ? n_kblocks : (d->max_k + kpi - 1) / kpi;
  // Pick the key-split count minimising a makespan estimate in units of one
  // iteration tile of one workgroup: (rounds of workgroups over all slots) x
  // (tiles per workgroup + 2 for pipeline fill and epilogue), plus, with
  // more than one split, the combine launch (~2) and its traffic: the
  // partial bytes relative to the K/V bytes all slots stream per tile, which
  // matches the measured combine durations.
  const int64_t slots = 256LL * pp.bf.wg_per_cu;
  int64_t max_s = iters < 1 ? 1 : iters;
  const int64_t lds_cap = ba::max_splits_bf16(d->d, pp.bf.variant);
  if (max_s > lds_cap) max_s = lds_cap;
  int64_t best_s = 1;
  double best_cost = 1e300;
  const bool gated = shares >= 1;
  if (!gated) shares = 1;
  const bool persistent = gated && per_seq && pp.bf.variant == 3;
  auto comb_of = [&](int64_t se, int64_t it) {
    return se > 1 ? 2.0 + (double)se * it * pp.bf.rows_per_wg / ((double)kpi * slots) : 0.0;
  };
  // Workgroups with keys to stream.  In varlen mode the key counts are
  // device data, so a sequence is taken to hold about 0.65 of max_k keys
  // (the splits past its end exit at once); for the multi-branch batch's
  // prefixes (2048 .. 8192 keys) this picks the split whose busy workgroups
  // fit one round of slots.
  const bool varlen = d->cu_q != nullptr;
  auto busy = [&](int64_t it, int64_t se) {
    return varlen ? it * (int64_t)std::ceil(0.65 * (double)se) : it * se;
  };
  for (int64_t s = 1; s <= max_s; ++s) {
    const int64_t ci = (iters + s - 1) / s;
    const int64_t se = ci > 0 ? (iters + ci - 1) / ci : 1;
    double span = 0.0, wsum = 0.0;
    for (int k = shares; k >= 1; --k) {
      const int64_t it = (items * k + shares - 1) / shares;
      double term = (double)((busy(it, se) + slots - 1) / slots) * (double)(ci + 2);
      if (persistent) term += comb_of(se, it);
      span += term / k;
      wsum += 1.0 / k;
    }
    if (gated) {
      span += 0.5 * (persistent ? 1.0 : (double)((items * se + slots - 1) / slots));
      wsum += 1.0;
    }
    const double comb = persistent ? 0.0 : comb_of(se, items);
    const double cost = span / wsum + comb;
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best_s = se;
    }
  }
  int64_t chunk_iters = (iters + best_s - 1) / best_s;
  if (chunk_iters < 1) chunk_iters = 1;
  if (listed) {
    if (chunk_iters > 64) chunk_iters = 64;
    pp.chunk = (int)chunk_iters;
    pp.n_splits = iters > 0 ? (int)((iters + chunk_iters - 1) / chunk_iters) : 1;
    return pp;
  }
  pp.chunk = (int)(chunk_iters * kpi);
  pp.n_splits = d->max_k > 0 ? (int)((d->max_k + pp.chunk - 1) / pp.chunk) : 1;
  if (pp.n_splits < 1) pp.n_splits = 1;
  return pp;
}

// Workspace: [partial A f32 [splits][entries][d]][partial L f32 [splits][entries]].
// Workspace of a split plan: partial A [splits][entries][d] f32, then
// partial L [splits][entries] f32.
// A gated fused step (bf16, valid cache, some prefix keys) always writes
// split partials, even with one split, so that a prefix workgroup whose wait
// for the gate gave up cannot overwrite a reused head's cache: the combine
// pass decides.  (With no prefix keys the result, A = 0 and L = -inf, does not
// depend on the decision.)
bool partial_always(const ba_attn_desc* d, bool gated_fused) {
  return gated_fused && d->dtype == BA_BF16 && d->max_k > 0;
}

size_t prefix_ws_bytes(const ba_attn_desc* d, const PrefixPlan& pp, bool gated_fused = false) {
  if (pp.n_splits <= 1 && !partial_always(d, gated_fused)) return 0;
  const size_t entries = (size_t)d->n_seq * d->max_q * d->hq;
  return (size_t)pp.n_splits * entries * (d->d + 1) * sizeof(float);
}

ba::AttnParams base_params(const ba_attn_desc* d, const AttnShape& sh) {
  ba::AttnParams p{};
  p.q = d->q;
  p.k = d->k;
  p.v = d->v;
  p.qs0 = d->q_stride[0];
  p.qs1 = d->q_stride[1];
  p.qs2 = d->q_stride[2];
  p.ks0 = d->k_stride[0];
  p.ks1 = d->k_stride[1];
  p.ks2 = d->k_stride[2];
  p.vs0 = d->v_stride[0];
  p.vs1 = d->v_stride[1];
  p.vs2 = d->v_stride[2];
  p.cu_q = d->cu_q;
  p.cu_k = d->cu_k;
  p.n_seq = d->n_seq;
  p.hq = d->hq;
  p.hkv = d->hkv;
  p.group = sh.group;
  p.max_q = d->max_q;
  p.max_k = d->max_k;
  p.scale_log2 = sh.scale * 1.44269504088896340736f;
  return p;
}

}  // namespace

extern "C" {

const char* ba_last_error(void) { return g_err.c_str(); }

int32_t ba_version(void) { return (1 << 16) | 0; }

namespace {

// Recomputing shares the split planner averages over for a gated fused step
// (valid cache): per head for the cosine gate, per sequence for the count
// gates; 1 otherwise.
constexpr int kMaxShares = 8;

// Shares for a gate that decides per sequence: one per sequence, at most
// kMaxShares.
int seq_shares(int n_seq) { return n_seq < 1 ? 1 : (n_seq < kMaxShares ? n_seq : kMaxShares); }

// 0 (ungated) unless the call is a gated fused step with a valid cache.
int gate_shares(const ba::GateParams* gate, const ba_attn_desc* desc) {
  if (!gate || !desc->decision) return 0;
  return gate->mode == BA_GATE_COSINE ? kMaxShares : seq_shares(desc->n_seq);
}

// Whether a gated fused step decides per sequence (count gates).
bool gate_per_seq(const ba::GateParams* gate) { return gate && gate->mode != BA_GATE_COSINE; }

}  // namespace

// Covers every plan a descriptor can get (ungated, and the gated fused
// step's, whose split count depends on the gate mode).
size_t ba_prefix_attn_workspace(const ba_attn_desc* desc) {
  AttnShape sh;
  if (check_desc(desc, &sh) != BA_OK) return 0;
  size_t need = 0;
  const int plans[3][2] = {{0, 0}, {seq_shares(desc->n_seq), 1}, {kMaxShares, 0}};   // (shares, per sequence)
  for (const auto& pl : plans) {
    const size_t b = prefix_ws_bytes(desc, plan_prefix(desc, sh.group, -1, pl[0], pl[1] != 0), pl[0] > 0);
    if (b > need) need = b;
  }
  return need;
}

namespace {

// Prefix attention, optionally followed by the merge with a precomputed
// in-block part (a_in != NULL).
ba_status prefix_impl(const ba_attn_desc* desc, float* a_out, float* l_out, const float* a_in,
                      const float* l_in, float* a_full, float* l_full, void* workspace,
                      size_t workspace_bytes, hipStream_t stream, ba::AttnParams* block = nullptr,
                      const ba_attn_desc* block_desc = nullptr, const ba::GateParams* gate = nullptr,
                      const int32_t* kblocks = nullptr, int n_kblocks = -1, const int32_t* cu_rows = nullptr,
                      const int32_t* rows = nullptr, bool dry_run = false) {
  AttnShape sh;
  ba_status st = check_desc(desc, &sh);
  if (st != BA_OK) return st;
  if (desc->n_seq == 0 || desc->max_q == 0) return BA_OK;
  if (!a_out || !l_out) return fail(BA_ERR_NULL, "a_out and l_out are required");
  const bool merge = a_in != nullptr || l_in != nullptr || a_full != nullptr || l_full != nullptr;
  if (merge && (!a_in || !l_in || !a_full))
    return fail(BA_ERR_NULL, "the merge needs a_in, l_in and a_full");
  if (merge && (!aligned16(a_in) || !aligned16(a_full) || !aligned16(a_out)))
    return fail(BA_ERR_UNSUPPORTED, "a_out, a_in and a_full must be 16-byte aligned");
  const PrefixPlan pp = plan_prefix(desc, sh.group, kblocks ? n_kblocks : -1, kblocks ? 0 : gate_shares(gate, desc),
                                    !kblocks && gate_per_seq(gate));
  // a gated fused step's prefix workgroups may give up waiting for the gate:
  // their results then go through the split workspace (see prefix_ws_bytes)
  const bool always_partial = partial_always(desc, gate != nullptr && desc->decision != nullptr);
  const size_t need = prefix_ws_bytes(desc, pp, always_partial);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(BA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
  if ((int64_t)pp.n_splits * pp.row_tiles * desc->n_seq * desc->hkv > 0x7fffff00LL)
    return fail(BA_ERR_UNSUPPORTED, "too many workgroups");
  // (the 256-row kernel's staged epilogue indexes (split, row, head)
  // entries with 32-bit integers)
  if (desc->dtype == BA_BF16 && pp.bf.variant == 3 &&
      (int64_t)pp.n_splits * desc->n_seq * desc->max_q * desc->hq > 0x7fffffffLL)
    return fail(BA_ERR_UNSUPPORTED, "too many (split, row, head) entries");
  ba::AttnParams p = base_params(desc, sh);
  p.decision = desc->decision;
  p.chunk = pp.chunk;
  p.n_splits = pp.n_splits;
  p.row_tiles = pp.row_tiles;
  p.a = a_out;
  p.l = l_out;
  p.kblocks = kblocks;
  p.n_kblocks = kblocks ? n_kblocks : 0;
  if (rows) {
    p.cu_q = cu_rows;
    p.q_rows = rows;
  }
  if (gate) {
    p.ready = gate->ready;
    p.ready_stride = gate->ready_stride;
    p.spin_limit = gate->spin_limit;
    p.gave_up = gate->gave_up;
    p.gate_mode = gate->mode;
    p.gate_tau = gate->tau;
  }
  if (block && desc->dtype != BA_F32) {
    // the in-block part rides on the same launch, in the prefix plan's shape
    // (the float32 kernel has no row tiles: one wave per row and head)
    const int brows = sh.group * block_desc->max_q;
    block->row_tiles = (brows + pp.bf.rows_per_wg - 1) / pp.bf.rows_per_wg;
    if ((int64_t)block->row_tiles * block_desc->n_seq * block_desc->hkv > 0x7fffff00LL)
      return fail(BA_ERR_UNSUPPORTED, "too many workgroups");
  }
  if (dry_run) return BA_OK;
  hipError_t err;
  if (desc->dtype == BA_F32 || (pp.n_splits == 1 && !always_partial)) {
    p.mode = ba::kPrefixFinal;
  } else {
    const size_t entries = (size_t)desc->n_seq * desc->max_q * desc->hq;
    p.mode = ba::kPrefixPartial;
    p.ws_a = static_cast<float*>(workspace);
    p.ws_l = p.ws_a + (size_t)pp.n_splits * entries * desc->d;
  }
  err = desc->dtype == BA_F32 ? ba::launch_attn_f32(p, desc->d, stream)
                              : ba::launch_attn_bf16(pp.bf, p, block, desc->d, stream, gate);
  if (err == hipSuccess && block && desc->dtype == BA_F32) err = ba::launch_attn_f32(*block, desc->d, stream);
  if (err != hipSuccess) return hip_status(err, "prefix attention");
  if (p.mode != ba::kPrefixPartial && !merge) return BA_OK;
  // One pass combines the split partials across many workgroups (the
  // combine needs the whole chip's bandwidth, not one workgroup's) and, when
  // asked, merges A_out/L_out (fresh, or cached for reused heads) with
  // A_in/L_in into A_full/L_full.
  if (merge) {
    p.a_cache = a_in;
    p.l_cache = l_in;
    p.a_full = a_full;
    p.l_full = l_full;
  }
  return hip_status(ba::launch_combine(p, desc->d, stream), merge ? "prefix merge" : "split combine");
}

}  // namespace

namespace {

// Key-block list mode is for the dense bf16 prefix kernels.
ba_status check_sparse(const ba_attn_desc* desc, int32_t n_blocks) {
  AttnShape sh;
  const ba_status st = check_desc(desc, &sh);
  if (st != BA_OK) return st;
  if (desc->dtype != BA_BF16) return fail(BA_ERR_UNSUPPORTED, "key-block lists need bf16");
  if (desc->cu_q || desc->cu_k) return fail(BA_ERR_UNSUPPORTED, "key-block lists are for dense prefixes");
  const int64_t n_max = ((int64_t)desc->max_k + ba::kBlockKeys - 1) / ba::kBlockKeys;
  if (n_blocks < 0 || n_blocks > n_max)
    return fail(BA_ERR_SHAPE, "n_blocks %d out of [0, %lld]", n_blocks, (long long)n_max);
  return BA_OK;
}

}  // namespace

size_t ba_sparse_prefix_attn_workspace(const ba_attn_desc* desc, int32_t n_blocks) {
  if (check_sparse(desc, n_blocks) != BA_OK) return 0;
  AttnShape sh;
  check_desc(desc, &sh);
  if (n_blocks == 0) {
    ba_attn_desc e = *desc;
    e.max_k = 0;
    return prefix_ws_bytes(&e, plan_prefix(&e, sh.group));
  }
  return prefix_ws_bytes(desc, plan_prefix(desc, sh.group, n_blocks));
}

ba_status ba_sparse_prefix_attn(const ba_attn_desc* desc, const int32_t* blocks, int32_t n_blocks, float* a_out,
                                float* l_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  const ba_status st = check_sparse(desc, n_blocks);
  if (st != BA_OK) return st;
  if (n_blocks == 0) {
    // no key selected: the attention of an empty key set (A = 0, L = -inf)
    ba_attn_desc e = *desc;
    e.max_k = 0;
    return prefix_impl(&e, a_out, l_out, nullptr, nullptr, nullptr, nullptr, workspace, workspace_bytes, stream);
  }
  if (!blocks) return fail(BA_ERR_NULL, "blocks is NULL");
  return prefix_impl(desc, a_out, l_out, nullptr, nullptr, nullptr, nullptr, workspace, workspace_bytes, stream,
                     nullptr, nullptr, nullptr, blocks, n_blocks);
}

ba_status ba_prefix_attn(const ba_attn_desc* desc, float* a_out, float* l_out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  return prefix_impl(desc, a_out, l_out, nullptr, nullptr, nullptr, nullptr, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Scratch of ba_prefix_attn_noalloc: the split-KV partials of one call, in a
// file-scope device array.  Each GPU the library runs on holds its own copy
// until the process ends.  In host code the array's name is only a host-side
// stand-in, never a device address: the address is looked up once per device
// (with that device current) through hipGetSymbolAddress and kept in
// g_scratch_dev, which is what kernels receive.
constexpr size_t kStaticScratchBytes = BA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on first use).
ba_status static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(BA_ERR_UNSUPPORTED, "device %d is beyond the %d devices the static scratch covers", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return BA_OK;
}

}  // namespace

extern "C" {

ba_status ba_prefix_attn_noalloc(const ba_attn_desc* desc, float* a_out, float* l_out, hipStream_t stream) {
  g_err.clear();
  AttnShape sh;
  const ba_status st = check_desc(desc, &sh);
  if (st != BA_OK) return st;
  // the same plan (and so the same kernels and results) as ba_prefix_attn
  const size_t need = prefix_ws_bytes(desc, plan_prefix(desc, sh.group));
  if (need > kStaticScratchBytes)
    return fail(BA_ERR_WORKSPACE,
                "this call needs %zu bytes of split scratch; the static scratch holds %zu (use ba_prefix_attn "
                "with a workspace)", need, kStaticScratchBytes);
  void* ws = nullptr;
  if (need > 0 && desc->n_seq > 0 && desc->max_q > 0) {
    const ba_status s2 = static_scratch(&ws);
    if (s2 != BA_OK) return s2;
  }
  return prefix_impl(desc, a_out, l_out, nullptr, nullptr, nullptr, nullptr, ws, ws ? kStaticScratchBytes : 0,
                     stream);
}

ba_status ba_prefix_attn_rows(const ba_attn_desc* desc, const int32_t* cu_rows, const int32_t* rows, float* a_out,
                              float* l_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  AttnShape sh;
  const ba_status st = check_desc(desc, &sh);
  if (st != BA_OK) return st;
  if (desc->cu_q || desc->cu_k) return fail(BA_ERR_UNSUPPORTED, "row lists are for dense descriptors");
  if (desc->decision) return fail(BA_ERR_SHAPE, "the descriptor's decision must be NULL (the row list selects)");
  if (desc->n_seq > 0 && desc->max_q > 0 && (!cu_rows || !rows))
    return fail(BA_ERR_NULL, "cu_rows and rows are required");
  return prefix_impl(desc, a_out, l_out, nullptr, nullptr, nullptr, nullptr, workspace, workspace_bytes, stream,
                     nullptr, nullptr, nullptr, nullptr, -1, cu_rows, rows);
}

ba_status ba_prefix_attn_merge(const ba_attn_desc* desc, float* a_out, float* l_out, const float* a_in,
                               const float* l_in, float* a_full, float* l_full, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  if (!a_in || !l_in || !a_full) return fail(BA_ERR_NULL, "a_in, l_in and a_full are required");
  return prefix_impl(desc, a_out, l_out, a_in, l_in, a_full, l_full, workspace, workspace_bytes, stream);
}

namespace {

// Prefix part and in-block part in one launch (with the gate, if given, in
// the same launch), then the combine-and-merge pass.
ba_status split_impl(const ba_attn_desc* prefix, const ba_attn_desc* block, float* a_out, float* l_out,
                     float* a_in, float* l_in, float* a_full, float* l_full, void* workspace,
                     size_t workspace_bytes, hipStream_t stream, const ba::GateParams* gate,
                     bool dry_run = false) {
  AttnShape sp, sb;
  ba_status st = check_desc(prefix, &sp);
  if (st != BA_OK) return st;
  st = check_desc(block, &sb);
  if (st != BA_OK) return st;
  if (prefix->dtype != block->dtype || prefix->n_seq != block->n_seq || prefix->hq != block->hq ||
      prefix->hkv != block->hkv || prefix->d != block->d || prefix->max_q != block->max_q ||
      sp.scale != sb.scale || sp.varlen != sb.varlen || prefix->q != block->q || prefix->cu_q != block->cu_q)
    return fail(BA_ERR_SHAPE, "prefix and block descriptors must share dtype, shapes, scale, q and cu_q");
  if (!a_in || !l_in || !a_full) return fail(BA_ERR_NULL, "a_in, l_in and a_full are required");
  if (prefix->n_seq == 0 || prefix->max_q == 0) return BA_OK;
  ba::AttnParams pb = base_params(block, sb);
  pb.decision = nullptr;
  pb.mode = ba::kBlock;
  pb.chunk = block->max_k > 0 ? block->max_k : 1;
  pb.n_splits = 1;
  pb.a = a_in;
  pb.l = l_in;
  return prefix_impl(prefix, a_out, l_out, a_in, l_in, a_full, l_full, workspace, workspace_bytes, stream, &pb,
                     block, gate, nullptr, -1, nullptr, nullptr, dry_run);
}

}  // namespace

ba_status ba_split_attn(const ba_attn_desc* prefix, const ba_attn_desc* block, float* a_out, float* l_out,
                        float* a_in, float* l_in, float* a_full, float* l_full, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  return split_impl(prefix, block, a_out, l_out, a_in, l_in, a_full, l_full, workspace, workspace_bytes, stream,
                    nullptr);
}

ba_status ba_block_attn(const ba_attn_desc* desc, const float* a_cache, const float* l_cache, float* a_in,
                        float* l_in, float* a_full, float* l_full, hipStream_t stream) {
  g_err.clear();
  AttnShape sh;
  ba_status st = check_desc(desc, &sh);
  if (st != BA_OK) return st;
  if ((a_cache == nullptr) != (l_cache == nullptr))
    return fail(BA_ERR_NULL, "a_cache and l_cache must both be given or both be NULL");
  if ((a_full || l_full) && !a_cache) return fail(BA_ERR_NULL, "a_full / l_full need the cache to merge with");
  if (!a_in && !l_in && !a_full && !l_full) return fail(BA_ERR_NULL, "no output given");
  if (desc->n_seq == 0 || desc->max_q == 0) return BA_OK;
  ba::AttnParams p = base_params(desc, sh);
  p.decision = nullptr;
  p.mode = ba::kBlock;
  p.chunk = desc->max_k > 0 ? desc->max_k : 1;
  p.n_splits = 1;
  p.a = a_in;
  p.l = l_in;
  p.a_cache = a_cache;
  p.l_cache = l_cache;
  p.a_full = a_full;
  p.l_full = l_full;
  if (desc->dtype == BA_F32) return hip_status(ba::launch_attn_f32(p, desc->d, stream), "block attention (f32)");
  const int rows = sh.group * desc->max_q;
  const ba::Bf16Plan bf = ba::plan_bf16(desc->d, rows, desc->max_k, false);
  if (bf.variant == 3 && (int64_t)desc->n_seq * desc->max_q * desc->hq > 0x7fffffffLL)
    return fail(BA_ERR_UNSUPPORTED, "too many (row, head) entries");   // (32-bit entry indexes)
  p.row_tiles = (rows + bf.rows_per_wg - 1) / bf.rows_per_wg;
  if ((int64_t)p.row_tiles * desc->n_seq * desc->hkv > 0x7fffff00LL)
    return fail(BA_ERR_UNSUPPORTED, "too many workgroups");
  return hip_status(ba::launch_attn_bf16(bf, p, nullptr, desc->d, stream), "block attention");
}

ba_status ba_lse_merge(int64_t rows, int32_t d, const float* a1, const float* l1, const float* a2,
                       const float* l2, float* a, float* l, hipStream_t stream) {
  g_err.clear();
  if (rows < 0) return fail(BA_ERR_SHAPE, "rows %lld is negative", (long long)rows);
  if (d < 4 || d > 1024 || d % 4) return fail(BA_ERR_UNSUPPORTED, "d %d (must be a multiple of 4 in [4, 1024])", d);
  if (rows == 0) return BA_OK;
  if (!a1 || !l1 || !a2 || !l2 || !a) return fail(BA_ERR_NULL, "a1, l1, a2, l2 and a are required");
  if (!aligned16(a1) || !aligned16(a2) || !aligned16(a))
    return fail(BA_ERR_UNSUPPORTED, "a1, a2 and a must be 16-byte aligned");
  if ((rows + (256 / (d / 4)) - 1) / (256 / (d / 4)) > 0x7fffffffLL) return fail(BA_ERR_SHAPE, "too many rows");
  ba::MergeParams p{rows, d, a1, l1, a2, l2, a, l};
  return hip_status(ba::launch_merge(p, stream), "lse merge");
}

size_t ba_reuse_gate_workspace(const ba_gate_desc* g) {
  if (!g || g->n_seq < 0 || g->hq < 1 || g->n_blk < 1 || g->d < 1) return 0;
  return ba::gate_workspace_bytes(g->mode, g->n_seq, g->hq, g->n_blk, g->d);
}

namespace {

// Validates a gate call and fills its launch parameters.
ba_status gate_params(const ba_gate_desc* g, int32_t* m_count, double* cos, uint8_t* decision, void* workspace,
                      size_t workspace_bytes, ba::GateParams* out) {
  if (!g) return fail(BA_ERR_NULL, "gate descriptor is NULL");
  if (g->mode != BA_GATE_COUNT && g->mode != BA_GATE_COSINE && g->mode != BA_GATE_COUNT_CUM &&
      g->mode != BA_GATE_ROWS)
    return fail(BA_ERR_SHAPE, "unknown gate mode %d", g->mode);
  if (g->dtype != BA_BF16 && g->dtype != BA_F32) return fail(BA_ERR_DTYPE, "unknown dtype %d", g->dtype);
  if (g->n_seq < 0 || g->n_blk < 1 || g->hq < 1 || g->d < 1)
    return fail(BA_ERR_SHAPE, "sizes n_seq %d, n_blk %d, hq %d, d %d", g->n_seq, g->n_blk, g->hq, g->d);
  if (g->n_seq > 65535 || g->n_blk > 0x7fffffff / 2) return fail(BA_ERR_UNSUPPORTED, "too many sequences");
  if (!decision) return fail(BA_ERR_NULL, "decision is required");
  const bool count = g->mode != BA_GATE_COSINE;   // count, cumulative count or rows
  if (count && !m_count) return fail(BA_ERR_NULL, "m_count is required in count mode");
  if (g->mode == BA_GATE_COUNT_CUM && !g->since_refresh)
    return fail(BA_ERR_NULL, "since_refresh is required in cumulative count mode");
  if (g->mode == BA_GATE_ROWS && (g->k_cur || g->k_prev || g->v_cur || g->v_prev))
    return fail(BA_ERR_SHAPE, "the rows gate reads Q only (k and v must be NULL)");
  if (count && g->n_blk > 65535) return fail(BA_ERR_UNSUPPORTED, "count gate supports n_blk <= 65535");
  if (count && !g->upd_mask) {
    if (!g->q_cur || !g->q_prev) return fail(BA_ERR_NULL, "q_cur and q_prev are required");
    if ((g->k_cur == nullptr) != (g->k_prev == nullptr) || (g->v_cur == nullptr) != (g->v_prev == nullptr))
      return fail(BA_ERR_NULL, "k_cur/k_prev and v_cur/v_prev must be given in pairs");
    if ((g->k_cur || g->v_cur) && (g->hkv < 1 || g->hq % g->hkv))
      return fail(BA_ERR_SHAPE, "hkv %d must divide hq %d", g->hkv, g->hq);
  }
  if (!count) {
    if (!g->q_cur || !g->q_prev) return fail(BA_ERR_NULL, "q_cur and q_prev are required");
    if (g->hq > 65535) return fail(BA_ERR_UNSUPPORTED, "hq > 65535");
  }
  for (int a = 0; a < 3; ++a)
    if (g->q_stride[a] < 0 || g->kv_stride[a] < 0) return fail(BA_ERR_SHAPE, "negative stride");
  const size_t need = ba::gate_workspace_bytes(g->mode, g->n_seq, g->hq, g->n_blk, g->d);
  if (!workspace || workspace_bytes < need)
    return fail(BA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
  ba::GateParams& p = *out;
  p = ba::GateParams{};
  p.mode = g->mode;
  p.esize = esize_of(g->dtype);
  p.n_seq = g->n_seq;
  p.n_blk = g->n_blk;
  p.hq = g->hq;
  p.hkv = g->hkv;
  p.d = g->d;
  p.q_cur = g->q_cur;
  p.q_prev = g->q_prev;
  p.qs0 = g->q_stride[0];
  p.qs1 = g->q_stride[1];
  p.qs2 = g->q_stride[2];
  p.k_cur = g->k_cur;
  p.k_prev = g->k_prev;
  p.v_cur = g->v_cur;
  p.v_prev = g->v_prev;
  p.ks0 = g->kv_stride[0];
  p.ks1 = g->kv_stride[1];
  p.ks2 = g->kv_stride[2];
  p.upd_mask = count ? g->upd_mask : nullptr;
  p.tau = g->tau;
  p.gamma = g->gamma;
  p.cache_valid = g->cache_valid ? 1 : 0;
  p.since = g->mode == BA_GATE_COUNT_CUM ? g->since_refresh : nullptr;
  p.pos_per_wg = 1;
  p.spin_limit = g->wait_polls == 0 ? kGateSpinLimit : (g->wait_polls < 0 ? 0 : g->wait_polls);
  p.gave_up = g->gave_up;
  p.chunks = count ? 1 : ba::gate_cos_chunks(g->n_blk, g->d);
  bool v16 = (g->d * p.esize) % 16 == 0;
  const void* ptrs[6] = {g->q_cur, g->q_prev, g->k_cur, g->k_prev, g->v_cur, g->v_prev};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) v16 = false;
  for (int a = 0; a < 3; ++a) {
    if ((g->q_stride[a] * p.esize) % 16) v16 = false;
    if ((g->k_cur || g->v_cur) && (g->kv_stride[a] * p.esize) % 16) v16 = false;
  }
  p.vec16 = v16 ? 1 : 0;
  p.m_count = count ? m_count : nullptr;
  p.cos = count ? nullptr : cos;
  p.decision = decision;
  p.ws_int = static_cast<int32_t*>(workspace);
  const size_t nbh = (size_t)g->n_seq * g->hq;
  p.ws_dbl = reinterpret_cast<double*>(static_cast<char*>(workspace) + ((nbh * sizeof(int32_t) + 15) & ~(size_t)15));
  return BA_OK;
}

// A fused call's gate workspace: the gate's own, then kReadyCopies copies of
// the per-sequence ready words (each copy n_seq ints rounded up to a
// 128-byte line).
size_t ready_stride_ints(const ba_gate_desc* g) { return ((size_t)g->n_seq + 31) & ~(size_t)31; }

size_t fused_gate_ws_bytes(const ba_gate_desc* g) {
  const size_t own = ba::gate_workspace_bytes(g->mode, g->n_seq, g->hq, g->n_blk, g->d);
  return ((own + 127) & ~(size_t)127) + ba::kReadyCopies * ready_stride_ints(g) * sizeof(int32_t);
}

}  // namespace

ba_status ba_reuse_gate(const ba_gate_desc* g, int32_t* m_count, double* cos, uint8_t* decision, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  ba::GateParams p;
  const ba_status st = gate_params(g, m_count, cos, decision, workspace, workspace_bytes, &p);
  if (st != BA_OK) return st;
  if (g->n_seq == 0) return BA_OK;
  return hip_status(ba::launch_gate(p, stream), "reuse gate");
}

size_t ba_gated_split_attn_gate_workspace(const ba_gate_desc* g) {
  if (!g || g->n_seq < 0 || g->hq < 1 || g->n_blk < 1 || g->d < 1) return 0;
  return fused_gate_ws_bytes(g);
}

ba_status ba_gated_split_attn(const ba_gate_desc* gate, int32_t* m_count, double* cos, uint8_t* decision,
                              void* gate_workspace, size_t gate_workspace_bytes, const ba_attn_desc* prefix,
                              const ba_attn_desc* block, float* a_out, float* l_out, float* a_in, float* l_in,
                              float* a_full, float* l_full, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  g_err.clear();
  if (!prefix || !block) return fail(BA_ERR_NULL, "attention descriptor is NULL");
  ba::GateParams gp;
  ba_status st = gate_params(gate, m_count, cos, decision, gate_workspace, gate_workspace_bytes, &gp);
  if (st != BA_OK) return st;
  if (gate_workspace_bytes < fused_gate_ws_bytes(gate))
    return fail(BA_ERR_WORKSPACE, "gate workspace of %zu bytes needed, %zu given", fused_gate_ws_bytes(gate),
                gate_workspace_bytes);
  if (gate->n_seq != prefix->n_seq || gate->hq != prefix->hq || gate->n_blk != prefix->max_q ||
      gate->dtype != prefix->dtype)
    return fail(BA_ERR_SHAPE, "gate and attention descriptors must share n_seq, hq, block size and dtype");
  if (prefix->decision) return fail(BA_ERR_SHAPE, "the prefix descriptor's decision must be NULL (the gate's is used)");
  if (gate->mode == BA_GATE_ROWS)
    return fail(BA_ERR_UNSUPPORTED, "the rows gate feeds ba_prefix_attn_rows, not a fused step");
  // The prefix part is gated by this call's decisions only when the cache
  // is valid; otherwise every head recomputes and nothing waits.
  ba_attn_desc pd = *prefix;
  pd.decision = gate->cache_valid ? decision : nullptr;
  if (prefix->dtype == BA_F32 || prefix->n_seq == 0 || prefix->max_q == 0) {
    // no fused launch for the float32 kernel: the gate, then the split pass,
    // whose arguments are all checked before the gate is enqueued
    st = split_impl(&pd, block, a_out, l_out, a_in, l_in, a_full, l_full, workspace, workspace_bytes, stream,
                    nullptr, /*dry_run=*/true);
    if (st != BA_OK) return st;
    if (prefix->n_seq > 0) {
      const hipError_t e = ba::launch_gate(gp, stream);
      if (e != hipSuccess) return hip_status(e, "reuse gate");
    }
    return split_impl(&pd, block, a_out, l_out, a_in, l_in, a_full, l_full, workspace, workspace_bytes, stream,
                      nullptr);
  }
  const size_t own = ba::gate_workspace_bytes(gate->mode, gate->n_seq, gate->hq, gate->n_blk, gate->d);
  gp.ready = reinterpret_cast<int32_t*>(static_cast<char*>(gate_workspace) + ((own + 127) & ~(size_t)127));

  gp.ready_stride = (int)ready_stride_ints(gate);
  return split_impl(&pd, block, a_out, l_out, a_in, l_in, a_full, l_full, workspace, workspace_bytes, stream, &gp);
}

ba_status ba_kl_lock(int32_t n, int64_t vocab, int32_t dtype, const void* logits_cur, const void* logits_prev,
                     int64_t row_stride, const uint8_t* eligible, float eps, float* kl, uint8_t* locked,
                     hipStream_t stream) {
  g_err.clear();
  if (n < 0 || vocab < 1) return fail(BA_ERR_SHAPE, "n %d and vocab %lld", n, (long long)vocab);
  if (dtype != BA_BF16 && dtype != BA_F32) return fail(BA_ERR_DTYPE, "unknown dtype %d", dtype);
  if (row_stride < vocab) return fail(BA_ERR_SHAPE, "row_stride %lld < vocab %lld", (long long)row_stride,
                                      (long long)vocab);
  if (!kl && !locked) return fail(BA_ERR_NULL, "no output given (kl and locked are both NULL)");
  if (n == 0) return BA_OK;
  if (!logits_cur || !logits_prev) return fail(BA_ERR_NULL, "logits_cur and logits_prev are required");
  if (!(eps >= 0.0f)) return fail(BA_ERR_SHAPE, "eps must be >= 0");
  ba::KlParams p{};
  p.n = n;
  p.vocab = vocab;
  p.stride = row_stride;
  p.esize = esize_of(dtype);
  p.vec = aligned16(logits_cur) && aligned16(logits_prev) && (row_stride * p.esize) % 16 == 0 ? 1 : 0;
  p.cur = logits_cur;
  p.prev = logits_prev;
  p.eligible = eligible;
  p.eps = eps;
  p.kl = kl;
  p.locked = locked;
  return hip_status(ba::launch_kl_lock(p, stream), "kl lock");
}

ba_status ba_varlen_pack(int32_t n_branch, const int32_t* block_sizes_host, const uint8_t* locked,
                         int32_t* cu_seqlens_q, int32_t* gather_idx, int32_t* total, int32_t dtype, int32_t h,
                         int32_t d, const void* q_src, const int64_t q_src_stride[2], void* q_packed,
                         hipStream_t stream) {
  g_err.clear();
  if (n_branch < 0 || n_branch > ba::kMaxBranches)
    return fail(BA_ERR_SHAPE, "n_branch %d out of [0, %d]", n_branch, ba::kMaxBranches);
  if (n_branch > 0 && !block_sizes_host) return fail(BA_ERR_NULL, "block_sizes_host is NULL");
  if (!cu_seqlens_q || !total) return fail(BA_ERR_NULL, "cu_seqlens_q and total are required");
  int32_t starts[ba::kMaxBranches + 1];
  int64_t run = 0;
  starts[0] = 0;
  for (int b = 0; b < n_branch; ++b) {
    if (block_sizes_host[b] < 0) return fail(BA_ERR_SHAPE, "block_sizes_host[%d] = %d is negative", b, block_sizes_host[b]);
    run += block_sizes_host[b];
    if (run > 0x7fffffff) return fail(BA_ERR_SHAPE, "total block size overflows int32");
    starts[b + 1] = (int32_t)run;
  }
  const int n_total = (int)run;
  if (n_total > 0 && (!locked || !gather_idx)) return fail(BA_ERR_NULL, "locked and gather_idx are required");
  if ((q_src == nullptr) != (q_packed == nullptr))
    return fail(BA_ERR_NULL, "q_src and q_packed must both be given or both be NULL");
  int es = 2;
  bool v16 = false;
  if (q_src) {
    if (dtype != BA_BF16 && dtype != BA_F32) return fail(BA_ERR_DTYPE, "unknown dtype %d", dtype);
    if (h < 1 || d < 1) return fail(BA_ERR_SHAPE, "h %d and d %d must be >= 1", h, d);
    if (!q_src_stride) return fail(BA_ERR_NULL, "q_src_stride is NULL");
    if (q_src_stride[0] < 0 || q_src_stride[1] < 0) return fail(BA_ERR_SHAPE, "negative stride");
    es = esize_of(dtype);
    if ((d * es) % 2) return fail(BA_ERR_SHAPE, "row bytes must be even");
    v16 = (d * es) % 16 == 0 && aligned16(q_src) && aligned16(q_packed) && (q_src_stride[0] * es) % 16 == 0 &&
          (q_src_stride[1] * es) % 16 == 0;
  }
  ba::PackParams p{};
  p.n_branch = n_branch;
  p.n_total = n_total;
  p.locked = locked;
  p.cu = cu_seqlens_q;
  p.gather = gather_idx;
  p.total = total;
  p.esize = es;
  p.h = h;
  p.d = d;
  p.q_src = q_src;
  p.qs0 = q_src ? q_src_stride[0] : 0;
  p.qs1 = q_src ? q_src_stride[1] : 0;
  p.q_packed = q_packed;
  p.vec16 = v16 ? 1 : 0;
  return hip_status(ba::launch_pack(p, starts, stream), "varlen pack");
}

}  // extern "C"
