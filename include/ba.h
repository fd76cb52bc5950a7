/*
 * ba.h - cached split attention for block diffusion, MI355X (gfx950) library.
 *
 * The step this library computes (FlashBlock summary, gist.science/es/paper/
 * 2602.05305, section 2 "Metodologia: FlashBlock", "Mecanismo Central"): the
 * active block's queries attend over a static out-of-block KV prefix, giving
 * an output A_out and its natural log-normaliser L_out = log Z_out, and over
 * the changing in-block tokens, giving A_in and L_in.  The two are combined by
 * the log-space merge
 *     m = max(L_out, L_in)
 *     A_full = (e^{L_out-m} A_out + e^{L_in-m} A_in) / (e^{L_out-m} + e^{L_in-m})
 * and L_full = m + log(e^{L_out-m} + e^{L_in-m}).  A_out/L_out are cached
 * across denoising steps and reused under a gate ("Estrategias de
 * Reutilizacion Adaptativa"): reuse when the number of updated tokens is
 * below tau, or, per head, when the head's similarity exceeds gamma.  Queries
 * of several branches can be packed into one variable-length buffer
 * (BlockBatch summary, gist.science/fr/paper/2605.29233, "Methodologie",
 * "Optimisation Systeme"); locked positions issue no query but stay attended
 * as keys (SURELOCK summary, gist.science/es/paper/2602.06412, section 2).
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is DEVICE memory owned by the caller unless its
 *     name ends in _host.  The library allocates nothing, frees nothing and
 *     never synchronises the stream: all work is enqueued on `stream`.
 *   - Arguments are validated on the host before anything is launched; on a
 *     non-OK status nothing was enqueued and ba_last_error() describes why.
 *     Device-resident metadata (cu_seqlens monotone and within bounds, lock
 *     flags in {0,1}) is the caller's contract and is not checked.
 *   - Element strides are in elements, never bytes; the last (head_dim) axis
 *     is always contiguous.  Row-major "[R, H, d]" means element (r, h, c) at
 *     (r*H + h)*d + c.
 *   - Results are bitwise reproducible: no floating-point atomics are used
 *     and the work split is a pure function of the shapes.
 *   - Calls are reentrant; concurrent calls on different streams that share a
 *     workspace race.
 */
#ifndef BA_H
#define BA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BA_OK = 0,
  BA_ERR_NULL = 1,        /* a required pointer is NULL                     */
  BA_ERR_SHAPE = 2,       /* inconsistent or out-of-range sizes / strides  */
  BA_ERR_DTYPE = 3,       /* unknown dtype                                 */
  BA_ERR_UNSUPPORTED = 4, /* valid request the library does not implement  */
  BA_ERR_WORKSPACE = 5,   /* workspace missing or too small                */
  BA_ERR_HIP = 6          /* a HIP launch reported an error                */
} ba_status;

typedef enum { BA_BF16 = 0, BA_F32 = 1 } ba_dtype;

typedef enum { BA_GATE_COUNT = 0, BA_GATE_COSINE = 1, BA_GATE_COUNT_CUM = 2, BA_GATE_ROWS = 3 } ba_gate_mode;

/*
 * Attention descriptor shared by ba_prefix_attn and ba_block_attn.
 *
 * Dense mode (cu_q == NULL and cu_k == NULL): n_seq sequences, each with
 *   max_q query rows and max_k keys.  Query row i of sequence b, head h is
 *   q + b*q_stride[0] + i*q_stride[1] + h*q_stride[2]; key j of KV head g is
 *   k + b*k_stride[0] + j*k_stride[1] + g*k_stride[2] (v likewise).
 * Varlen mode (cu_q and cu_k both non-NULL, device int32[n_seq+1], each
 *   starting at 0 and non-decreasing): sequence b owns query rows
 *   cu_q[b] .. cu_q[b+1]-1 and keys cu_k[b] .. cu_k[b+1]-1; the row index is
 *   used directly with stride [1] (stride [0] is ignored).  max_q / max_k
 *   must bound every sequence's row / key count (they size the launch).
 * Grouped-query attention: query head h reads KV head h / (hq / hkv).
 * Output layout of every A (float32) is [R, hq, d] and of every L (float32)
 *   [R, hq], where R = n_seq*max_q in dense mode (row b*max_q + i) and the
 *   packed row index cu_q[b] + i in varlen mode.
 * decision: optional device uint8[n_seq, hq] as written by ba_reuse_gate;
 *   1 = keep the cached A_out/L_out of that (sequence, head), 0 = recompute.
 *   NULL = recompute everything.  Only ba_prefix_attn reads it.
 * Limits (BA_ERR_UNSUPPORTED beyond them): n_seq * hkv <= 65535 in dense
 *   mode; hq / hkv * max_q <= 2^30 rows per KV head; on the 256-row kernel
 *   (more than 192 rows per KV head) key splits x n_seq x max_q x hq < 2^31.
 */
typedef struct ba_attn_desc {
  int32_t dtype;            /* ba_dtype of q, k and v                          */
  int32_t n_seq;            /* sequences (batch) or branches                   */
  int32_t hq, hkv;          /* query heads, KV heads; hq % hkv == 0            */
  int32_t d;                /* head dim: 64 or 128                             */
  int32_t max_q, max_k;     /* rows / keys per sequence (bounds in varlen)     */
  float scale;              /* softmax scale; <= 0 selects 1/sqrt(d)           */
  const void* q; int64_t q_stride[3];
  const void* k; int64_t k_stride[3];
  const void* v; int64_t v_stride[3];
  const int32_t* cu_q;      /* device, varlen only                             */
  const int32_t* cu_k;      /* device, varlen only                             */
  const uint8_t* decision;  /* device, optional (prefix only)                  */
} ba_attn_desc;

/*
 * Out-of-block (prefix) attention, FlashBlock "Mecanismo Central": for every
 * (sequence, query head) whose decision is 0 (or all, if decision is NULL),
 * A_out[i] = sum_j softmax_j(s q_i.k_j) v_j over the sequence's prefix keys
 * and L_out[i] = log sum_j exp(s q_i.k_j), written in place into the caller's
 * cache a_out [R, hq, d] / l_out [R, hq].  Entries of (sequence, head) pairs
 * with decision 1 are left untouched (the cached values stay).  An empty
 * prefix gives A_out = 0, L_out = -inf.
 * The key range is split across workgroups; partial results go to
 * `workspace`, whose size ba_prefix_attn_workspace() returns (0 means none is
 * needed and workspace may be NULL).  That size covers every call that takes
 * this descriptor's prefix workspace (a per-head gated fused step may split
 * the keys more finely than the other calls).  The workspace needs no
 * initialisation; calls that overlap in time must not share one.
 */
size_t ba_prefix_attn_workspace(const ba_attn_desc* desc);
ba_status ba_prefix_attn(const ba_attn_desc* desc, float* a_out, float* l_out,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * ba_prefix_attn for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Identical to ba_prefix_attn (same split plan, kernels and results) except
 * that the split-KV partials go to a static scratch array inside the library
 * instead of a caller workspace; the call allocates nothing and calls no
 * allocating routine.  Each GPU holds one such array of
 * BA_NOALLOC_SCRATCH_BYTES (64 MiB) from the library's first use on it until
 * the process ends; a call whose split partials would not fit
 * (ba_prefix_attn_workspace(desc) larger than that) returns
 * BA_ERR_WORKSPACE and enqueues nothing.  The array of the device current at
 * the call is used.  Every call on a GPU shares that GPU's array, so calls
 * that overlap in time on one GPU (different streams, or graphs replayed
 * concurrently) race; calls in one stream's order do not.  Nothing in the
 * array needs to start at zero: a call writes every partial it reads.
 */
#define BA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ba_status ba_prefix_attn_noalloc(const ba_attn_desc* desc, float* a_out, float* l_out, hipStream_t stream);

/*
 * Partial refresh of the cached out-of-block part (FlashBlock, section 2,
 * "Estrategias de Reutilizacion Adaptativa": the cache is reused while few
 * block tokens change; here the rows that did change are recomputed and the
 * rest kept).  A_out/L_out of a query row depend only on that row's Q and
 * the static prefix K/V, so recomputing exactly the rows whose Q changed
 * since the cache was written gives the same cache as recomputing all rows,
 * at the cost of the changed rows.
 *   desc: a dense prefix descriptor (cu_q = cu_k = decision = NULL) over the
 *     whole block Q [n_seq, max_q, hq, d] and the prefix K/V, as for
 *     ba_prefix_attn.
 *   cu_rows: device int32[n_seq + 1]; rows: device int32[cu_rows[n_seq]]:
 *     the rows of sequence b are rows[j] - b * max_q for j in
 *     [cu_rows[b], cu_rows[b + 1]) (at most max_q of them) -- exactly the
 *     cu_seqlens_q and gather_idx that ba_varlen_pack writes for n_seq
 *     branches of max_q positions each, with locked = "row is current"
 *     (ba_reuse_gate in BA_GATE_ROWS mode writes that mask).  A row index
 *     out of range is clamped into the sequence (a wrong result, never an
 *     access outside Q or the cache).
 *   a_out / l_out: the dense cache [n_seq * max_q, hq, d] / [n_seq * max_q,
 *     hq]; only the listed rows are written.
 *   workspace: ba_prefix_attn_workspace(desc) bytes.
 * Errors as for ba_prefix_attn.
 */
ba_status ba_prefix_attn_rows(const ba_attn_desc* desc, const int32_t* cu_rows, const int32_t* rows, float* a_out,
                              float* l_out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Prefix attention over listed key blocks only, for the sparse-attention
 * residual reuse of FlashBlock (section 2, "Estrategias de Reutilizacion
 * Adaptativa", the point on sparse attention; "Contribuciones Clave" 3): the
 * keys a sparse attention leaves out are treated as the out-of-block set,
 * whose contribution is computed once and cached, while the selected keys
 * are attended fresh; the two results are joined by the merge equation
 * (ba_lse_merge), and merging the results of a list and of its complement
 * gives ba_prefix_attn over the whole prefix.
 * Exactly ba_prefix_attn (decision gating, outputs, workspace rules) with
 * the keys of (sequence b, KV head g) restricted to the blocks
 *     blocks[(b*hkv + g)*n_blocks + i], i < n_blocks   (device int32),
 * block j being keys [64*j, min(64*j + 64, max_k)).  Dense bf16 only
 * (cu_q, cu_k NULL); 0 <= n_blocks <= ceil(max_k / 64).  The indices of one
 * list must be distinct and in [0, ceil(max_k/64)); this is device data, the
 * caller's contract: an index out of range is clamped into it (a wrong
 * result, never an access outside K/V).  n_blocks == 0 gives A = 0,
 * L = -inf.  The workspace is sized by ba_sparse_prefix_attn_workspace.
 */
size_t ba_sparse_prefix_attn_workspace(const ba_attn_desc* desc, int32_t n_blocks);
ba_status ba_sparse_prefix_attn(const ba_attn_desc* desc, const int32_t* blocks, int32_t n_blocks,
                                float* a_out, float* l_out, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * Prefix attention fused with the log-space merge of FlashBlock "Mecanismo
 * Central", for a step that computes the in-block part first (for example
 * ba_block_attn with a_in/l_in outputs, concurrently with the reuse gate):
 * exactly ba_prefix_attn, and then for every (row, query head)
 *   A_full, L_full = merge(A_out, L_out, A_in, L_in)
 * by the equation in this header's preamble, where A_out/L_out are the values
 * just computed or, for (sequence, head) pairs whose decision is 1, the
 * cached ones already in a_out/l_out.  a_in/l_in and a_full/l_full are
 * float32 [R, hq, d] / [R, hq] with R as for a_out (rows past a sequence's
 * length in varlen mode are not touched); l_full may be NULL.  The
 * workspace is the one ba_prefix_attn_workspace() sizes for the same
 * descriptor.  Errors as for ba_prefix_attn; a_in, l_in, a_full are required.
 */
ba_status ba_prefix_attn_merge(const ba_attn_desc* desc, float* a_out, float* l_out,
                               const float* a_in, const float* l_in, float* a_full, float* l_full,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The whole split attention of one denoising step, FlashBlock "Mecanismo
 * Central": the out-of-block part (desc `prefix`, gated by prefix->decision
 * exactly as in ba_prefix_attn) and the in-block part (desc `block`, as
 * ba_block_attn with a_in/l_in outputs) run in one launch, since neither
 * depends on the other; then one pass combines the prefix's key splits and
 * merges: A_full, L_full = merge(A_out, L_out, A_in, L_in), A_out/L_out
 * fresh or, for reused heads, the cached ones.  Equivalent to ba_block_attn
 * (a_in, l_in) followed by ba_prefix_attn_merge, in two launches instead of
 * three.  The two descriptors must share dtype, n_seq, hq, hkv, d, max_q,
 * scale, q and cu_q (they differ in k/v, their strides, cu_k and max_k).
 * a_in, l_in, a_full are required, l_full may be NULL; the workspace is the
 * one ba_prefix_attn_workspace(prefix) sizes.
 */
ba_status ba_split_attn(const ba_attn_desc* prefix, const ba_attn_desc* block, float* a_out, float* l_out,
                        float* a_in, float* l_in, float* a_full, float* l_full, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/*
 * In-block attention with the fused log-space merge, FlashBlock "Mecanismo
 * Central": every query row attends over all of its sequence's block keys
 * with no mask (the block is bidirectional), giving A_in / L_in.  If a_cache
 * and l_cache are both non-NULL, they are merged with A_in/L_in by the
 * equation in this header's preamble into a_full / l_full.  Outputs are
 * optional individually (NULL = not written) but at least one must be given;
 * a_full / l_full require the cache.  desc->decision is ignored.
 */
ba_status ba_block_attn(const ba_attn_desc* desc, const float* a_cache, const float* l_cache,
                        float* a_in, float* l_in, float* a_full, float* l_full,
                        hipStream_t stream);

/*
 * Standalone log-space merge of two partial results over disjoint key sets
 * (FlashBlock "Mecanismo Central", the merge equation): for each of `rows`
 * rows, a1/a2 are float32 [rows, d], l1/l2 float32 [rows]; writes a [rows, d]
 * and, if l is non-NULL, l [rows] = m + log(e^{l1-m} + e^{l2-m}).  A side with
 * L = -inf weighs nothing; both -inf gives A = 0, L = -inf.  In-place use
 * (a == a1 or a == a2, l == l1 or l == l2) is allowed.
 */
ba_status ba_lse_merge(int64_t rows, int32_t d, const float* a1, const float* l1,
                       const float* a2, const float* l2, float* a, float* l,
                       hipStream_t stream);

/*
 * Reuse gate descriptor (FlashBlock "Estrategias de Reutilizacion
 * Adaptativa").  Block tensors are [n_seq, n_blk, heads, d] addressed with
 * the given (sequence, position, head) element strides.
 *   BA_GATE_COUNT: M_b = number of block positions p of sequence b whose Q,
 *     K or V row (any head, any element) differs bitwise between *_cur and
 *     *_prev; if upd_mask (device uint8[n_seq, n_blk]) is non-NULL, M_b is
 *     instead the number of its nonzero entries and no tensor is read.
 *     decision[b, h] = cache_valid && M_b < tau, the same for every head.
 *   BA_GATE_COSINE: per (b, h), the cosine of the head's whole block Q (all
 *     n_blk*d values) against the previous step's, accumulated in float64:
 *     cos = dot / (sqrt(|q|^2) * sqrt(|q'|^2)), a zero norm giving cos = 0
 *     and recompute; decision[b, h] = cache_valid && cos > gamma.
 *   BA_GATE_COUNT_CUM: as BA_GATE_COUNT, but M_b counts the positions
 *     updated at any step since sequence b's cache was last written (the
 *     count "since the last refresh", a variant the pages leave open next to
 *     the per-step count).  since_refresh (device uint8[n_seq, n_blk]) holds
 *     that set between calls: a position is marked when it changes, and all
 *     of b's marks are cleared when decision[b, :] = 0 (the cache is
 *     rewritten this step).  A call with cache_valid == 0 clears every mark,
 *     so the array needs no initialisation before a block's first step.
 *   BA_GATE_ROWS: per block position (partial refresh, see
 *     ba_prefix_attn_rows): decision is uint8[n_seq, n_blk] with
 *     decision[b, p] = cache_valid && position p's Q row (every head) is
 *     bitwise unchanged (or upd_mask[b, p] == 0); m_count[b] = the number
 *     of changed positions.  Only Q is read (k_* and v_* must be NULL);
 *     tau is not used.
 *   Ties (M == tau, cos == gamma) recompute; cache_valid == 0 recomputes all.
 */
typedef struct ba_gate_desc {
  int32_t mode;             /* ba_gate_mode                                    */
  int32_t dtype;            /* ba_dtype of the block tensors                   */
  int32_t n_seq, n_blk, hq, hkv, d;
  const void* q_cur; const void* q_prev; int64_t q_stride[3];
  const void* k_cur; const void* k_prev;        /* count mode; both or neither */
  const void* v_cur; const void* v_prev;        /* count mode; both or neither */
  int64_t kv_stride[3];
  const uint8_t* upd_mask;  /* count mode, optional                            */
  int32_t tau;
  double gamma;
  int32_t cache_valid;      /* 0 = no cache yet (first step of a block)        */
  uint8_t* since_refresh;   /* BA_GATE_COUNT_CUM state; NULL in other modes    */
  /* ba_gated_split_attn only (ignored by ba_reuse_gate):                     */
  int32_t wait_polls;       /* polls of a prefix workgroup's bounded wait for
                               the gate: 0 = the default (about a second),
                               > 0 = that many, < 0 = none (every gated prefix
                               workgroup gives up at once; for failure-
                               handling tests)                                 */
  int32_t* gave_up;         /* optional device int32: one is added per prefix
                               workgroup that gave up waiting                  */
} ba_gate_desc;

/*
 * Workspace for ba_reuse_gate: it must be zero-filled before its first use;
 * every call leaves it zero-filled again when it completes.
 */
size_t ba_reuse_gate_workspace(const ba_gate_desc* g);
/*
 * Outputs: m_count int32[n_seq] (count mode; may be NULL in cosine mode),
 * cos float64[n_seq, hq] (cosine mode, optional), decision uint8[n_seq, hq]
 * (required; 1 = reuse).
 */
ba_status ba_reuse_gate(const ba_gate_desc* g, int32_t* m_count, double* cos,
                        uint8_t* decision, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * One denoising step with the reuse gate in the same launch as the split
 * attention (FlashBlock, section 2: the gate of "Estrategias de
 * Reutilizacion Adaptativa" decides, per head, whether the out-of-block part
 * of "Mecanismo Central" is recomputed or reused).  Equivalent to
 * ba_reuse_gate(gate, ...) followed by ba_split_attn(prefix', block, ...),
 * where prefix' is *prefix with decision = (gate->cache_valid ? decision :
 * NULL), but in two launches instead of three: the gate's workgroups come
 * first in the attention launch and each gated prefix workgroup waits (with
 * agent-scope loads, bounded) until the gate has written its sequence's
 * decisions; the in-block part does not wait.  With a valid cache the key
 * split is planned for a step that recomputes part of the heads or
 * sequences, so it can be finer than ba_split_attn's; the outputs then agree
 * with that sequence of calls up to the rounding of the split-KV combine.
 *   gate, m_count, cos, decision: as for ba_reuse_gate; gate->n_seq, hq,
 *     dtype and n_blk must equal prefix->n_seq, hq, dtype and max_q.
 *   gate_workspace: ba_gated_split_attn_gate_workspace(gate) bytes, zero-
 *     filled before first use; every call that returns BA_OK leaves it zero
 *     again.  A call whose launch fails leaves it undefined: zero it again.
 *   A prefix workgroup whose wait for the gate runs out (gate->wait_polls;
 *     by default after about a second, far beyond the gate's running time)
 *     computes its heads into the split workspace instead, and the combine
 *     pass, which runs after the gate has finished, applies the gate's
 *     decisions to them: the outputs do not depend on whether a wait gave
 *     up.  Such workgroups are counted in *gate->gave_up when it is given.
 *   With a valid cache (bf16) the prefix part always goes through the split
 *     workspace, even with a single key split, so `workspace` is required;
 *     ba_prefix_attn_workspace(prefix) covers it.
 *   prefix->decision must be NULL; everything else as for ba_split_attn.
 * The float32 dtype runs the two calls in sequence (no fused launch).
 */
size_t ba_gated_split_attn_gate_workspace(const ba_gate_desc* gate);
ba_status ba_gated_split_attn(const ba_gate_desc* gate, int32_t* m_count, double* cos, uint8_t* decision,
                              void* gate_workspace, size_t gate_workspace_bytes,
                              const ba_attn_desc* prefix, const ba_attn_desc* block, float* a_out,
                              float* l_out, float* a_in, float* l_in, float* a_full, float* l_full,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Lock criterion of SURELOCK ("Deteccion de Convergencia"): for each of n
 * token rows, the KL divergence of the token's current posterior over the
 * vocabulary from the previous step's,
 *     kl[r] = KL(p || q),  p = softmax(logits_cur[r, :]), q = softmax(logits_prev[r, :]),
 * with natural logs; a row with eligible[r] != 0 (or every row, if eligible
 * is NULL) locks once kl[r] < eps: locked[r] is set to 1, and never cleared
 * (a locked token stays locked).  The lock flags feed ba_varlen_pack.
 *   logits_cur, logits_prev: device [n, vocab] of dtype (bf16 or float32),
 *     rows row_stride elements apart (row_stride >= vocab).  A -inf logit is
 *     allowed (that entry has probability 0); a row whose q is 0 where p is
 *     not has KL = +inf.
 *   kl: optional device float32 [n]; locked: optional device uint8 [n]
 *     (read and written); at least one must be given.
 * Sums are accumulated in float64 from float32 exponentials; the result is
 * reproducible and within about 1e-6 of the exact KL for vocabularies of a
 * few hundred thousand entries.
 */
ba_status ba_kl_lock(int32_t n, int64_t vocab, int32_t dtype, const void* logits_cur,
                     const void* logits_prev, int64_t row_stride, const uint8_t* eligible,
                     float eps, float* kl, uint8_t* locked, hipStream_t stream);

/*
 * Varlen packing of unlocked query positions across branches (BlockBatch
 * "Optimisation Systeme"; SURELOCK "Accion de Bloqueo").  Branch b owns block
 * positions sum(block_sizes_host[:b]) .. ; a position with locked[p] != 0
 * issues no query.  Writes, branch-major with ascending position:
 *   cu_seqlens_q int32[n_branch+1]: exclusive prefix sum of unlocked counts;
 *   gather_idx int32[N] (N = sum of block sizes): packed row r -> position,
 *     entries r >= total set to -1;
 *   total int32[1];
 *   q_packed [N, h, d] (contiguous, dtype of q_src): row r < total is the
 *     q_src row gather_idx[r]; rows >= total are left untouched.
 * q_src rows are addressed with (position, head) element strides
 * q_src_stride[0..1].  q_src / q_packed may both be NULL to skip the gather.
 * 0 <= n_branch <= 512.
 */
ba_status ba_varlen_pack(int32_t n_branch, const int32_t* block_sizes_host,
                         const uint8_t* locked, int32_t* cu_seqlens_q, int32_t* gather_idx,
                         int32_t* total, int32_t dtype, int32_t h, int32_t d,
                         const void* q_src, const int64_t q_src_stride[2], void* q_packed,
                         hipStream_t stream);

/* Thread-local text of the last non-OK status ("" if none). */
const char* ba_last_error(void);

/* Library ABI version: (major << 16) | minor. */
int32_t ba_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BA_H */
