"""CPU fp64 oracle for cached split attention in block diffusion.

TEST INFRASTRUCTURE ONLY.  This module is the yardstick the GPU library is
checked against.  Only the tests, the smoke check and the benchmark's CPU
baseline leg may import it; the library itself never does, and this module
imports nothing from the library.  It is deliberately plain and slow: NumPy
float64, one (sequence, head) at a time, no blocking, fusion or reordering
beyond the definitions below.

Sources (gist.science summaries):
  [FB]  "Resumen Tecnico: FlashBlock" (es/paper/2602.05305), section 2
        "Metodologia: FlashBlock": "Mecanismo Central" (the in-block /
        out-of-block split, the cached A_out and L_out = log Z_out, and the
        log-space merge equation) and "Estrategias de Reutilizacion
        Adaptativa" (threshold gate tau on the count of updated tokens,
        per-head similarity gate gamma for video).
  [SL]  "Resumen Tecnico: SURELOCK" (es/paper/2602.06412), section 2,
        "Accion de Bloqueo" and "Mantenimiento de la Atencion Global": locked
        tokens issue no queries but stay attended through their cached K/V;
        "Deteccion de Convergencia": a token locks once the KL divergence of
        its posterior from the previous step's falls below a threshold.
  [BB]  "Resume Technique : BlockBatch" (fr/paper/2605.29233), "Methodologie",
        "Optimisation Systeme": unmasked query positions of all branches are
        packed into one variable-length buffer.
  [FB] also, in "Estrategias de Reutilizacion Adaptativa", sparse attention:
        the keys a sparse pass leaves out are the "out" set whose contribution
        is cached and merged with the fresh pass over the selected keys.

Readings of points the pages leave open (each is listed in the design notes):
  softmax scale s given by the caller (1/sqrt(d) by default); L is a natural
  log; the merged normaliser is L_full = m + log(e^{L1-m} + e^{L2-m}); an
  empty key set gives A = 0, L = -inf and weighs nothing in a merge; the
  prefix is fully visible and the block is bidirectional (no mask); query head
  h reads KV head h // (Hq/Hkv); "updated tokens" are block positions whose
  Q, K or V row (any head) differs bitwise from the previous step's; reuse iff
  count < tau, or iff cosine > gamma (ties recompute); the first step of a
  block always recomputes; the cosine is that of the head's whole block Q
  (Nb*d values) against the previous step's, a zero norm recomputes; packing
  is branch-major with ascending position.  Gate variants the pages leave
  open: a count of the positions updated since the last refresh (not only
  into this step); a partial refresh that recomputes exactly the rows whose Q
  changed.

Parity status: every function here is pinned by the CPU tests (closed forms,
mpmath brute force, the split/merge identity, integer schedules, hand-derived
worked examples).  The absolute outputs of the five synthetic workloads have
no printed reference values on the pages; they rest on those pins.
"""

from __future__ import annotations

import math

import numpy as np


# ----------------------------------------------------------------------------
# input decoding (the oracle's own; it shares no helper with the GPU path)
# ----------------------------------------------------------------------------

def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of a bf16 bit-pattern array or a float32 array."""
    if dtype == "bf16":
        u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# attention and the log-space merge
# ----------------------------------------------------------------------------

def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Softmax attention of query rows q[n, d] over keys k[m, d], values v[m, dv].

    [FB] Mecanismo Central: each part of the split yields an output A and its
    log-normaliser L = log Z, Z = sum_j exp(s * q . k_j).  Returns
    (A[n, dv], L[n]).  An empty key set gives A = 0 and L = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, m = q.shape[0], k.shape[0]
    if m == 0:
        return np.zeros((n, v.shape[1])), np.full(n, -np.inf)
    z = scale * (q @ k.T)                    # [n, m] scores
    mx = z.max(axis=1)                       # shift for exp; cancels in A
    e = np.exp(z - mx[:, None])
    zsum = e.sum(axis=1)
    a = (e @ v) / zsum[:, None]
    lse = mx + np.log(zsum)
    return a, lse


def merge(a1, l1, a2, l2):
    """Log-space merge of two partial results over disjoint key sets.

    [FB] Mecanismo Central, merge equation: with m = max(L1, L2),
    A = (e^{L1-m} A1 + e^{L2-m} A2) / (e^{L1-m} + e^{L2-m}).
    The merged log-normaliser is L = m + log(e^{L1-m} + e^{L2-m}) (reading:
    the pages print only A).  A side with L = -inf weighs nothing; both -inf
    gives A = 0, L = -inf.  a* have shape [..., dv], l* shape [...].
    """
    a1 = np.asarray(a1, dtype=np.float64)
    a2 = np.asarray(a2, dtype=np.float64)
    l1 = np.asarray(l1, dtype=np.float64)
    l2 = np.asarray(l2, dtype=np.float64)
    m = np.maximum(l1, l2)
    empty = np.isneginf(m)
    m_ref = np.where(empty, 0.0, m)
    w1 = np.where(np.isneginf(l1), 0.0, np.exp(l1 - m_ref))
    w2 = np.where(np.isneginf(l2), 0.0, np.exp(l2 - m_ref))
    den = w1 + w2
    safe = np.where(empty, 1.0, den)
    a = (w1[..., None] * a1 + w2[..., None] * a2) / safe[..., None]
    a = np.where(empty[..., None], 0.0, a)
    lse = np.where(empty, -np.inf, m_ref + np.log(safe))
    return a, lse


def merge_many(parts):
    """Fold merge() over a list of (A, L) pairs, left to right."""
    a, l = parts[0]
    for a2, l2 in parts[1:]:
        a, l = merge(a, l, a2, l2)
    return a, l


# ----------------------------------------------------------------------------
# reuse gates
# ----------------------------------------------------------------------------

def updated_positions(cur, prev) -> np.ndarray:
    """Per sequence, the block positions whose row changed bitwise.

    cur/prev: lists of arrays [B, Nb, H*, d] (Q, K, V of this step and the
    previous one), in their stored form (bf16 bit patterns or float32).
    Returns bool [B, Nb].  [FB] Estrategias de Reutilizacion Adaptativa counts
    "updated tokens"; reading: a token is updated when any element of its Q,
    K or V row, in any head, differs from the previous step's.
    """
    changed = None
    for c, p in zip(cur, prev):
        c = np.ascontiguousarray(c)
        p = np.ascontiguousarray(p)
        width = {2: np.uint16, 4: np.uint32, 8: np.uint64}[c.dtype.itemsize]
        diff = (c.view(width) != p.view(width)).reshape(c.shape[0], c.shape[1], -1).any(axis=2)
        changed = diff if changed is None else (changed | diff)
    return changed


def update_count(cur, prev) -> np.ndarray:
    """M_b: number of updated block positions of sequence b (int32 [B])."""
    return updated_positions(cur, prev).sum(axis=1).astype(np.int32)


def gate_count(m_count, tau: int, cache_valid: bool, hq: int) -> np.ndarray:
    """Threshold gate.  [FB] Estrategias de Reutilizacion Adaptativa: reuse the
    cached out-of-block attention when M < tau, otherwise recompute.
    Returns uint8 [B, Hq], 1 = reuse.  With no valid cache every entry is 0.
    """
    m_count = np.asarray(m_count)
    reuse = (m_count < tau) if cache_valid else np.zeros(m_count.shape, dtype=bool)
    return np.repeat(reuse[:, None], hq, axis=1).astype(np.uint8)


def cumulative_gates(changed, tau: int, hq: int):
    """Count gate on the positions updated since the cache was last written.

    [FB] Estrategias de Reutilizacion Adaptativa gates on a count of updated
    tokens; this is the variant where the count runs from the last refresh
    instead of the previous step (a reading the pages leave open).  Written
    from the definition: at step t, with r the latest step before t whose
    gate recomputed sequence b (none: r = 0), M_b(t) = the number of
    positions updated at any step s with r < s <= t; reuse iff the cache is
    valid (t > 1) and M_b(t) < tau.

    changed: list indexed by step t = 1..S (entry 0 unused) of bool [B, Nb],
    the positions updated in the transition into step t.  Returns a list
    indexed the same way of dicts with 'm' (int32 [B]) and 'decision'
    (uint8 [B, Hq]).
    """
    steps = len(changed) - 1
    B = changed[1].shape[0]
    out = [None]
    for t in range(1, steps + 1):
        m = np.zeros(B, dtype=np.int32)
        for b in range(B):
            r = 0
            for s_ in range(1, t):
                if out[s_]["decision"][b, 0] == 0:
                    r = s_
            union = np.zeros(changed[t].shape[1], dtype=bool)
            for s_ in range(r + 1, t + 1):
                union |= changed[s_][b]
            m[b] = int(union.sum())
        out.append(dict(m=m, decision=gate_count(m, tau, t > 1, hq)))
    return out


def rows_changed(q_cur, q_prev) -> np.ndarray:
    """Per sequence, the block positions whose Q row (any head) changed
    bitwise: the rows whose out-of-block part a partial refresh recomputes.
    A row's A_out/L_out depend only on its own query and the static prefix
    ([FB] Mecanismo Central), so the other rows' cached values are current.
    Returns bool [B, Nb]."""
    return updated_positions([q_cur], [q_prev])


def head_cosine(q_cur: np.ndarray, q_prev: np.ndarray):
    """Cosine similarity, per (sequence, head), of the head's block Q now vs.
    at the previous step, over all Nb*d values.

    [FB] Estrategias de Reutilizacion Adaptativa (video): a per-head
    similarity estimate; reading: this cosine.  Inputs are float64 values
    [B, Nb, H, d].  Every sum is math.fsum (correctly rounded); products of
    bf16 or fp32 values are exact in float64.  Returns (cos[B, H],
    zero[B, H]) where zero marks a head with a zero norm on either side
    (cos is then reported as 0).
    """
    B, _, H, _ = q_cur.shape
    cos = np.zeros((B, H))
    zero = np.zeros((B, H), dtype=bool)
    for b in range(B):
        for h in range(H):
            x = q_cur[b, :, h, :].ravel()
            y = q_prev[b, :, h, :].ravel()
            dot = math.fsum((x * y).tolist())
            nx = math.fsum((x * x).tolist())
            ny = math.fsum((y * y).tolist())
            if nx == 0.0 or ny == 0.0:
                zero[b, h] = True
                continue
            cos[b, h] = dot / (math.sqrt(nx) * math.sqrt(ny))
    return cos, zero


def gate_cosine(cos, zero, gamma: float, cache_valid: bool) -> np.ndarray:
    """Per-head gate.  [FB] Estrategias de Reutilizacion Adaptativa: only
    heads whose similarity exceeds gamma reuse the cache.  uint8 [B, H]."""
    if not cache_valid:
        return np.zeros(np.shape(cos), dtype=np.uint8)
    return ((np.asarray(cos) > gamma) & ~np.asarray(zero)).astype(np.uint8)


# ----------------------------------------------------------------------------
# varlen packing of unlocked queries
# ----------------------------------------------------------------------------

def kl_rows(logits_cur, logits_prev) -> np.ndarray:
    """Per row, KL(p || q) with p = softmax(cur row), q = softmax(prev row),
    natural logs, float64.  [SL] Deteccion de Convergencia: D_t = KL(p_t ||
    p_{t-1}) of each token's posterior over the vocabulary.  Entries with
    p = 0 contribute 0; q = 0 where p > 0 gives +inf."""
    x = np.asarray(logits_cur, dtype=np.float64)
    y = np.asarray(logits_prev, dtype=np.float64)
    out = np.empty(x.shape[0])
    for r in range(x.shape[0]):
        lp = x[r] - x[r].max()
        lp = lp - math.log(np.exp(lp).sum())
        lq = y[r] - y[r].max()
        lq = lq - math.log(np.exp(lq).sum())
        p = np.exp(lp)
        with np.errstate(invalid="ignore"):
            terms = np.where(p > 0, p * (lp - lq), 0.0)
        out[r] = terms.sum()
    return out


def lock_update(locked, eligible, kl, eps: float) -> np.ndarray:
    """[SL] Deteccion de Convergencia / Accion de Bloqueo: an eligible token
    locks once its KL falls below eps, and a locked token stays locked."""
    return (np.asarray(locked, dtype=bool) | (np.asarray(eligible, dtype=bool) & (kl < eps))).astype(np.uint8)


def varlen_pack(locked, block_sizes):
    """Pack the unlocked block positions of all branches into one buffer.

    [BB] Optimisation Systeme: the unmasked query positions of every active
    branch go into one variable-length buffer.  [SL] Accion de Bloqueo: a
    locked position issues no query.  Reading: branch-major, ascending
    position.  Returns (cu_seqlens int32[nb+1], gather_idx int32[total],
    total); gather_idx[r] is the global block position of packed row r.
    """
    locked = np.asarray(locked).astype(np.int64)
    bs = np.asarray(block_sizes, dtype=np.int64)
    starts = np.concatenate([[0], np.cumsum(bs)])
    cu = [0]
    gather = []
    for b in range(bs.size):
        for p in range(int(starts[b]), int(starts[b + 1])):
            if locked[p] == 0:
                gather.append(p)
        cu.append(len(gather))
    return (np.asarray(cu, dtype=np.int32), np.asarray(gather, dtype=np.int32), len(gather))


# ----------------------------------------------------------------------------
# one block's denoising schedule
# ----------------------------------------------------------------------------

def step_gates(sched):
    """Gate outputs for every step of a block schedule.

    Returns a list indexed by step t = 1..S (entry 0 unused) of dicts with
    'm' (int32 [B]), 'cos' (float64 [B, Hq] or None), 'decision' (uint8
    [B, Hq]).  Step 1 has no valid cache and recomputes everything.  gate
    "count" counts the positions updated into step t, "count_cum" those
    updated since the last refresh (cumulative_gates), "cosine" is the
    per-head similarity gate.
    """
    out = [None]
    if sched.gate == "count_cum":
        changed = [None] + [updated_positions([sched.q[t], sched.k[t], sched.v[t]],
                                              [sched.q[t - 1], sched.k[t - 1], sched.v[t - 1]])
                            for t in range(1, sched.steps + 1)]
        for g in cumulative_gates(changed, sched.tau, sched.hq)[1:]:
            out.append(dict(m=g["m"], cos=None, decision=g["decision"]))
        return out
    for t in range(1, sched.steps + 1):
        valid = t > 1
        m = update_count([sched.q[t], sched.k[t], sched.v[t]],
                         [sched.q[t - 1], sched.k[t - 1], sched.v[t - 1]])
        cos = None
        if sched.gate == "count":
            dec = gate_count(m, sched.tau, valid, sched.hq)
        else:
            cos, zero = head_cosine(to_f64(sched.q[t], sched.dtype),
                                    to_f64(sched.q[t - 1], sched.dtype))
            dec = gate_cosine(cos, zero, sched.gamma, valid)
        out.append(dict(m=m, cos=cos, decision=dec))
    return out


def refresh_steps(gates, steps: int) -> np.ndarray:
    """For each step t and (b, h), the latest step <= t that recomputed the
    prefix part (whose Q the cached A_out/L_out were built from)."""
    dec0 = gates[1]["decision"]
    last = np.zeros((steps + 1,) + dec0.shape, dtype=np.int64)
    cur = np.zeros(dec0.shape, dtype=np.int64)
    for t in range(1, steps + 1):
        cur = np.where(gates[t]["decision"] == 0, t, cur)
        last[t] = cur
    return last


def prefix_rows(sched, t_ref: int, b: int, h: int, rows=None):
    """(A_out, L_out) of query head h of sequence b over the prefix, with the
    block Q of step t_ref.  [FB] Mecanismo Central (out-of-block part)."""
    g = sched.hq // sched.hkv
    q = to_f64(sched.q[t_ref][b, :, h, :], sched.dtype)
    if rows is not None:
        q = q[rows]
    k = to_f64(sched.kp[b, h // g], sched.dtype)
    v = to_f64(sched.vp[b, h // g], sched.dtype)
    return attention(q, k, v, sched.scale)


def block_keys(blocks, lp: int, block_keys: int = 64) -> np.ndarray:
    """Key indices of a list of key blocks: block j is keys
    [block_keys*j, block_keys*(j+1)) clipped to the prefix length."""
    idx = [np.arange(block_keys * j, min(block_keys * (j + 1), lp)) for j in np.asarray(blocks, dtype=np.int64)]
    return np.concatenate(idx) if idx else np.zeros(0, dtype=np.int64)


def prefix_rows_in_blocks(sched, t_ref: int, b: int, h: int, blocks, rows=None):
    """(A, L) of query head h of sequence b over the prefix keys of the listed
    blocks only.  [FB] Estrategias de Reutilizacion Adaptativa, sparse
    attention: a sparse pass attends over the selected keys, and the
    unselected keys are the "out" set whose contribution is cached; both are
    plain attention over a key subset, joined by the Mecanismo Central merge."""
    g = sched.hq // sched.hkv
    q = to_f64(sched.q[t_ref][b, :, h, :], sched.dtype)
    if rows is not None:
        q = q[rows]
    sel = block_keys(blocks, sched.lp)
    k = to_f64(sched.kp[b, h // g][sel], sched.dtype)
    v = to_f64(sched.vp[b, h // g][sel], sched.dtype)
    return attention(q, k, v, sched.scale)


def block_rows(sched, t: int, b: int, h: int, rows=None):
    """(A_in, L_in) of query head h of sequence b over the block at step t,
    all Nb positions visible.  [FB] Mecanismo Central (in-block part)."""
    g = sched.hq // sched.hkv
    q = to_f64(sched.q[t][b, :, h, :], sched.dtype)
    if rows is not None:
        q = q[rows]
    k = to_f64(sched.k[t][b, :, h // g, :], sched.dtype)
    v = to_f64(sched.v[t][b, :, h // g, :], sched.dtype)
    return attention(q, k, v, sched.scale)


def run_block(sched, exact=False, partial=False):
    """The method on a whole block schedule, all rows of all heads.

    For each step: gate; for every (b, h) the gate sends to recompute,
    (A_out, L_out) over the prefix with the current Q replaces the cache
    ([FB] Mecanismo Central: the cache holds A_out and L_out from the last
    time they were computed); (A_in, L_in) over the block; A_full = merge.
    With partial=True the gate is per row instead (partial refresh): at
    step 1 every row is computed, afterwards exactly the rows whose Q
    changed from the previous step (rows_changed), in every head.
    Outputs use the library's row-major layout [B*Nb, Hq, d] / [B*Nb, Hq].
    With exact=True also returns the full attention over prefix + block with
    the current Q (for reporting how stale a reused cache is).
    """
    B, nb, hq, d = sched.B, sched.nb, sched.hq, sched.d
    gates = step_gates(sched)
    a_out = np.full((B, nb, hq, d), np.nan)
    l_out = np.full((B, nb, hq), np.nan)
    steps = [None]
    g = hq // sched.hkv
    for t in range(1, sched.steps + 1):
        dec = gates[t]["decision"]
        a_in = np.zeros((B, nb, hq, d))
        l_in = np.zeros((B, nb, hq))
        a_ex = np.zeros((B, nb, hq, d)) if exact else None
        if partial:
            redo = np.ones((B, nb), dtype=bool) if t == 1 else rows_changed(sched.q[t], sched.q[t - 1])
        for b in range(B):
            for h in range(hq):
                if partial:
                    rows = np.flatnonzero(redo[b])
                    if rows.size:
                        a_out[b, rows, h], l_out[b, rows, h] = prefix_rows(sched, t, b, h, rows)
                elif dec[b, h] == 0:
                    a_out[b, :, h], l_out[b, :, h] = prefix_rows(sched, t, b, h)
                a_in[b, :, h], l_in[b, :, h] = block_rows(sched, t, b, h)
                if exact:
                    q = to_f64(sched.q[t][b, :, h, :], sched.dtype)
                    kk = np.concatenate([to_f64(sched.kp[b, h // g], sched.dtype),
                                         to_f64(sched.k[t][b, :, h // g], sched.dtype)])
                    vv = np.concatenate([to_f64(sched.vp[b, h // g], sched.dtype),
                                         to_f64(sched.v[t][b, :, h // g], sched.dtype)])
                    a_ex[b, :, h], _ = attention(q, kk, vv, sched.scale)
        a_full, l_full = merge(a_out, l_out, a_in, l_in)
        rec = dict(gate=gates[t],
                   a_out=a_out.reshape(B * nb, hq, d).copy(),
                   l_out=l_out.reshape(B * nb, hq).copy(),
                   a_in=a_in.reshape(B * nb, hq, d), l_in=l_in.reshape(B * nb, hq),
                   a_full=a_full.reshape(B * nb, hq, d), l_full=l_full.reshape(B * nb, hq))
        if exact:
            rec["a_exact"] = a_ex.reshape(B * nb, hq, d)
        steps.append(rec)
    return steps


def run_varlen(batch, heads=None):
    """One step of the multi-branch varlen batch with a cold cache.

    Packed row r = (branch b, position p) attends over branch b's own prefix
    and over all of branch b's block positions, locked ones included ([SL]
    Mantenimiento de la Atencion Global); the two parts are merged ([FB]).
    Returns dict with the packing, and A_out/L_out/A_in/L_in/A_full/L_full
    in packed layout [total, H, d] / [total, H] (heads restricted to `heads`
    if given, other heads left NaN).
    """
    cu, gather, total = varlen_pack(batch.locked, batch.block_sizes)
    H, d = batch.h, batch.d
    heads = range(H) if heads is None else heads
    bstart = np.concatenate([[0], np.cumsum(batch.block_sizes)])
    pstart = np.concatenate([[0], np.cumsum(batch.prefix_lens)])
    res = {k: np.full((total, H, d), np.nan) for k in ("a_out", "a_in", "a_full")}
    res.update({k: np.full((total, H), np.nan) for k in ("l_out", "l_in", "l_full")})
    for b in range(batch.block_sizes.size):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        if r1 == r0:
            continue
        pos = gather[r0:r1]
        for h in heads:
            q = to_f64(batch.q[pos, h, :], batch.dtype)
            kp = to_f64(batch.kp[h, pstart[b]:pstart[b + 1]], batch.dtype)
            vp = to_f64(batch.vp[h, pstart[b]:pstart[b + 1]], batch.dtype)
            kb = to_f64(batch.k[bstart[b]:bstart[b + 1], h], batch.dtype)
            vb = to_f64(batch.v[bstart[b]:bstart[b + 1], h], batch.dtype)
            ao, lo = attention(q, kp, vp, batch.scale)
            ai, li = attention(q, kb, vb, batch.scale)
            af, lf = merge(ao, lo, ai, li)
            res["a_out"][r0:r1, h], res["l_out"][r0:r1, h] = ao, lo
            res["a_in"][r0:r1, h], res["l_in"][r0:r1, h] = ai, li
            res["a_full"][r0:r1, h], res["l_full"][r0:r1, h] = af, lf
    res.update(cu_seqlens=cu, gather_idx=gather, total=total)
    return res
