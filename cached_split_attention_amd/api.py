"""Python binding of the C-ABI in include/ba.h: same entry-point names, torch
tensors in, argument marshalling only.  Every step of the computation runs in
the HIP kernels of libba.so; nothing here computes.

Layout names used by the keyword `*_layout` arguments (last dim contiguous):
  "bshd"  [B, L, H, d]    "bhsd"  [B, H, L, d]    (dense)
  "thd"   [T, H, d]       "htd"   [H, T, d]       (varlen, with cu_seqlens)
"""

from __future__ import annotations

import ctypes

import torch

from ._lib import (AttnDesc, GateDesc, BA_BF16, BA_F32, BA_GATE_COUNT, BA_GATE_COSINE, BA_GATE_COUNT_CUM,
                   BA_GATE_ROWS, c_i64x2, check, lib)

__all__ = ["ba_prefix_attn_workspace", "ba_prefix_attn", "ba_prefix_attn_merge", "ba_split_attn",
           "ba_block_attn", "ba_lse_merge", "ba_reuse_gate_workspace", "ba_reuse_gate",
           "ba_gated_split_attn_gate_workspace", "ba_gated_split_attn", "ba_varlen_pack", "ba_version",
           "ba_sparse_prefix_attn_workspace", "ba_sparse_prefix_attn", "ba_kl_lock",
           "ba_prefix_attn_rows", "ba_prefix_attn_noalloc", "BA_GATE_COUNT", "BA_GATE_COSINE", "BA_GATE_COUNT_CUM", "BA_GATE_ROWS"]


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BA_BF16
    if t.dtype == torch.float32:
        return BA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on the GPU")


def _strides(t: torch.Tensor, layout: str):
    """(sequence, token, head) element strides and (n_seq, tokens, heads, d)."""
    if t.stride(-1) != 1:
        raise ValueError("the head-dim axis must be contiguous")
    s = t.stride()
    if layout == "bshd":
        return (s[0], s[1], s[2]), (t.shape[0], t.shape[1], t.shape[2], t.shape[3])
    if layout == "bhsd":
        return (s[0], s[2], s[1]), (t.shape[0], t.shape[2], t.shape[1], t.shape[3])
    if layout == "thd":
        return (0, s[0], s[1]), (None, t.shape[0], t.shape[1], t.shape[2])
    if layout == "htd":
        return (0, s[1], s[0]), (None, t.shape[1], t.shape[0], t.shape[2])
    raise ValueError(f"unknown layout {layout!r}")


def _desc(q, k, v, *, q_layout, kv_layout, cu_q, cu_k, max_q, max_k, scale, decision):
    _need_gpu(q, k, v, cu_q, cu_k, decision)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    varlen = cu_q is not None
    if varlen != (cu_k is not None):
        raise ValueError("cu_q and cu_k go together")
    qs, (qb, qn, hq, d) = _strides(q, q_layout)
    ks, (kb, kn, hkv, dk) = _strides(k, kv_layout)
    vs, (vb, vn, hv, dv) = _strides(v, kv_layout)
    if dk != d or dv != d or hv != hkv or vn != kn or vb != kb:
        raise ValueError("k / v shapes do not match q")
    if varlen:
        for c in (cu_q, cu_k):
            if c.dtype != torch.int32 or c.dim() != 1:
                raise TypeError("cu_seqlens must be 1-D int32")
        n_seq = cu_q.numel() - 1
        if cu_k.numel() != n_seq + 1:
            raise ValueError("cu_q and cu_k lengths differ")
        if max_q is None or max_k is None:
            raise ValueError("varlen mode needs max_q and max_k")
    else:
        n_seq = qb
        if kb != qb:
            raise ValueError("batch of q and k differ")
        max_q = qn if max_q is None else max_q
        max_k = kn if max_k is None else max_k
    if decision is not None and (decision.dtype != torch.uint8 or decision.numel() != n_seq * hq):
        raise ValueError("decision must be uint8 [n_seq, hq]")
    desc = AttnDesc()
    desc.dtype = _dtype(q)
    desc.n_seq, desc.hq, desc.hkv, desc.d = n_seq, hq, hkv, d
    desc.max_q, desc.max_k = int(max_q), int(max_k)
    desc.scale = 0.0 if scale is None else float(scale)
    desc.q, desc.k, desc.v = q.data_ptr(), k.data_ptr(), v.data_ptr()
    for i in range(3):
        desc.q_stride[i], desc.k_stride[i], desc.v_stride[i] = qs[i], ks[i], vs[i]
    desc.cu_q, desc.cu_k, desc.decision = _ptr(cu_q), _ptr(cu_k), _ptr(decision)
    # outputs: [n_seq*max_q, hq, d] dense, [packed rows, hq, d] varlen
    rows = qn if varlen else n_seq * desc.max_q
    return desc, rows


def _check_out(t, shape, dtype, name):
    if t is None:
        return
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} GPU tensor")
    if t.numel() < int(torch.Size(shape).numel()):
        raise ValueError(f"{name} holds {t.numel()} elements, {tuple(shape)} needed")


def ba_version() -> int:
    return lib().ba_version()


def ba_prefix_attn_workspace(q, k, v, *, q_layout="bshd", kv_layout="bhsd", cu_q=None, cu_k=None,
                             max_q=None, max_k=None, scale=None) -> int:
    desc, _ = _desc(q, k, v, q_layout=q_layout, kv_layout=kv_layout, cu_q=cu_q, cu_k=cu_k,
                    max_q=max_q, max_k=max_k, scale=scale, decision=None)
    return int(lib().ba_prefix_attn_workspace(ctypes.byref(desc)))


def ba_prefix_attn(q, k, v, a_out, l_out, workspace=None, *, q_layout="bshd", kv_layout="bhsd",
                   cu_q=None, cu_k=None, max_q=None, max_k=None, decision=None, scale=None,
                   stream=None):
    """Out-of-block attention into the cache (a_out [R, hq, d], l_out [R, hq])."""
    desc, rows = _desc(q, k, v, q_layout=q_layout, kv_layout=kv_layout, cu_q=cu_q, cu_k=cu_k,
                       max_q=max_q, max_k=max_k, scale=scale, decision=decision)
    _check_out(a_out, (rows, desc.hq, desc.d), torch.float32, "a_out")
    _check_out(l_out, (rows, desc.hq), torch.float32, "l_out")
    _need_gpu(workspace)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib().ba_prefix_attn(ctypes.byref(desc), _ptr(a_out), _ptr(l_out), _ptr(workspace), nbytes,
                               _stream(stream)))


def ba_prefix_attn_noalloc(q, k, v, a_out, l_out, *, q_layout="bshd", kv_layout="bhsd", cu_q=None, cu_k=None,
                           max_q=None, max_k=None, decision=None, scale=None, stream=None):
    """ba_prefix_attn with its split partials in the library's static per-GPU scratch
    (no workspace, no allocation; calls overlapping on one GPU race)."""
    desc, rows = _desc(q, k, v, q_layout=q_layout, kv_layout=kv_layout, cu_q=cu_q, cu_k=cu_k,
                       max_q=max_q, max_k=max_k, scale=scale, decision=decision)
    _check_out(a_out, (rows, desc.hq, desc.d), torch.float32, "a_out")
    _check_out(l_out, (rows, desc.hq), torch.float32, "l_out")
    check(lib().ba_prefix_attn_noalloc(ctypes.byref(desc), _ptr(a_out), _ptr(l_out), _stream(stream)))


def ba_prefix_attn_rows(q, k, v, cu_rows, rows, a_out, l_out, workspace=None, *, kv_layout="bhsd", scale=None,
                        stream=None):
    """Partial refresh: prefix attention for the listed block rows only (q [B, Nb, hq, d] dense;
    cu_rows int32 [B + 1] and rows int32 (global rows b*Nb + position) as ba_varlen_pack writes
    them), written into those rows of the cache a_out [B*Nb, hq, d] / l_out [B*Nb, hq].  The
    workspace is the one ba_prefix_attn_workspace(q, k, v) sizes."""
    desc, n_rows = _desc(q, k, v, q_layout="bshd", kv_layout=kv_layout, cu_q=None, cu_k=None,
                         max_q=None, max_k=None, scale=scale, decision=None)
    _need_gpu(cu_rows, rows, workspace)
    for t, nm in ((cu_rows, "cu_rows"), (rows, "rows")):
        if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
            raise TypeError(f"{nm} must be a contiguous 1-D int32 tensor")
    if cu_rows.numel() != desc.n_seq + 1:
        raise ValueError("cu_rows must have n_seq + 1 entries")
    _check_out(a_out, (n_rows, desc.hq, desc.d), torch.float32, "a_out")
    _check_out(l_out, (n_rows, desc.hq), torch.float32, "l_out")
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib().ba_prefix_attn_rows(ctypes.byref(desc), _ptr(cu_rows), _ptr(rows), _ptr(a_out), _ptr(l_out),
                                    _ptr(workspace), nbytes, _stream(stream)))


def _blocks(blocks, desc):
    _need_gpu(blocks)
    if blocks.dtype != torch.int32 or blocks.dim() != 3 or not blocks.is_contiguous() or \
            tuple(blocks.shape[:2]) != (desc.n_seq, desc.hkv):
        raise ValueError("blocks must be a contiguous int32 tensor [n_seq, hkv, n_blocks]")
    return int(blocks.shape[2])


def ba_sparse_prefix_attn_workspace(q, k, v, blocks, *, kv_layout="bhsd", scale=None) -> int:
    desc, _ = _desc(q, k, v, q_layout="bshd", kv_layout=kv_layout, cu_q=None, cu_k=None,
                    max_q=None, max_k=None, scale=scale, decision=None)
    return int(lib().ba_sparse_prefix_attn_workspace(ctypes.byref(desc), _blocks(blocks, desc)))


def ba_sparse_prefix_attn(q, k, v, blocks, a_out, l_out, workspace=None, *, kv_layout="bhsd",
                          decision=None, scale=None, stream=None):
    """Prefix attention over the listed key blocks (blocks: int32 [n_seq, hkv, n_blocks],
    block j = keys 64j .. 64j+63) into a_out [R, hq, d] / l_out [R, hq]; dense bf16."""
    desc, rows = _desc(q, k, v, q_layout="bshd", kv_layout=kv_layout, cu_q=None, cu_k=None,
                       max_q=None, max_k=None, scale=scale, decision=decision)
    n_blocks = _blocks(blocks, desc)
    _check_out(a_out, (rows, desc.hq, desc.d), torch.float32, "a_out")
    _check_out(l_out, (rows, desc.hq), torch.float32, "l_out")
    _need_gpu(workspace)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib().ba_sparse_prefix_attn(ctypes.byref(desc), _ptr(blocks), n_blocks, _ptr(a_out), _ptr(l_out),
                                      _ptr(workspace), nbytes, _stream(stream)))


def ba_prefix_attn_merge(q, k, v, a_out, l_out, a_in, l_in, a_full, l_full=None, workspace=None, *,
                         q_layout="bshd", kv_layout="bhsd", cu_q=None, cu_k=None, max_q=None, max_k=None,
                         decision=None, scale=None, stream=None):
    """ba_prefix_attn, then A_full/L_full = merge(A_out/L_out, A_in/L_in) for every row and head
    (A_out/L_out fresh, or cached for heads whose decision is 1)."""
    desc, rows = _desc(q, k, v, q_layout=q_layout, kv_layout=kv_layout, cu_q=cu_q, cu_k=cu_k,
                       max_q=max_q, max_k=max_k, scale=scale, decision=decision)
    for t, nm in ((a_out, "a_out"), (a_in, "a_in"), (a_full, "a_full")):
        _check_out(t, (rows, desc.hq, desc.d), torch.float32, nm)
    for t, nm in ((l_out, "l_out"), (l_in, "l_in")):
        _check_out(t, (rows, desc.hq), torch.float32, nm)
    if l_full is not None:
        _check_out(l_full, (rows, desc.hq), torch.float32, "l_full")
    _need_gpu(workspace)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib().ba_prefix_attn_merge(ctypes.byref(desc), _ptr(a_out), _ptr(l_out), _ptr(a_in), _ptr(l_in),
                                     _ptr(a_full), _ptr(l_full), _ptr(workspace), nbytes, _stream(stream)))


def ba_split_attn(q, kp, vp, k, v, a_out, l_out, a_in, l_in, a_full, l_full=None, workspace=None, *,
                  q_layout="bshd", kv_layout="bhsd", block_kv_layout="bshd", cu_q=None, cu_kp=None,
                  cu_k=None, max_q=None, max_kp=None, max_k=None, decision=None, scale=None, stream=None):
    """Prefix part (kp, vp; gated by decision) and in-block part (k, v) in one launch, then the
    split combine and the merge into a_full/l_full."""
    dp, rows = _desc(q, kp, vp, q_layout=q_layout, kv_layout=kv_layout, cu_q=cu_q, cu_k=cu_kp,
                     max_q=max_q, max_k=max_kp, scale=scale, decision=decision)
    db, _ = _desc(q, k, v, q_layout=q_layout, kv_layout=block_kv_layout, cu_q=cu_q, cu_k=cu_k,
                  max_q=max_q, max_k=max_k, scale=scale, decision=None)
    for t, nm in ((a_out, "a_out"), (a_in, "a_in"), (a_full, "a_full")):
        _check_out(t, (rows, dp.hq, dp.d), torch.float32, nm)
    for t, nm in ((l_out, "l_out"), (l_in, "l_in")):
        _check_out(t, (rows, dp.hq), torch.float32, nm)
    if l_full is not None:
        _check_out(l_full, (rows, dp.hq), torch.float32, "l_full")
    _need_gpu(workspace)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib().ba_split_attn(ctypes.byref(dp), ctypes.byref(db), _ptr(a_out), _ptr(l_out), _ptr(a_in),
                              _ptr(l_in), _ptr(a_full), _ptr(l_full), _ptr(workspace), nbytes,
                              _stream(stream)))


def ba_block_attn(q, k, v, *, a_cache=None, l_cache=None, a_in=None, l_in=None, a_full=None,
                  l_full=None, q_layout="bshd", kv_layout="bshd", cu_q=None, cu_k=None, max_q=None,
                  max_k=None, scale=None, stream=None):
    """In-block attention, optionally merged with the cached prefix part."""
    desc, rows = _desc(q, k, v, q_layout=q_layout, kv_layout=kv_layout, cu_q=cu_q, cu_k=cu_k,
                       max_q=max_q, max_k=max_k, scale=scale, decision=None)
    for t, n, shp in ((a_cache, "a_cache", (rows, desc.hq, desc.d)), (l_cache, "l_cache", (rows, desc.hq)),
                      (a_in, "a_in", (rows, desc.hq, desc.d)), (l_in, "l_in", (rows, desc.hq)),
                      (a_full, "a_full", (rows, desc.hq, desc.d)), (l_full, "l_full", (rows, desc.hq))):
        _check_out(t, shp, torch.float32, n)
    check(lib().ba_block_attn(ctypes.byref(desc), _ptr(a_cache), _ptr(l_cache), _ptr(a_in), _ptr(l_in),
                              _ptr(a_full), _ptr(l_full), _stream(stream)))


def ba_lse_merge(a1, l1, a2, l2, a, l=None, stream=None):
    """a = merge((a1, l1), (a2, l2)) row by row; a* [rows, d], l* [rows]."""
    _need_gpu(a1, l1, a2, l2, a, l)
    d = a1.shape[-1]
    rows = a1.numel() // d
    for t, n, shp in ((a1, "a1", (rows, d)), (a2, "a2", (rows, d)), (a, "a", (rows, d)),
                      (l1, "l1", (rows,)), (l2, "l2", (rows,)), (l, "l", (rows,))):
        _check_out(t, shp, torch.float32, n)
    check(lib().ba_lse_merge(rows, d, _ptr(a1), _ptr(l1), _ptr(a2), _ptr(l2), _ptr(a), _ptr(l),
                             _stream(stream)))


def _gate_desc(mode, q_cur, q_prev, k_cur, k_prev, v_cur, v_prev, upd_mask, tau, gamma, cache_valid,
               since_refresh=None, wait_polls=0, gave_up=None):
    _need_gpu(q_cur, q_prev, k_cur, k_prev, v_cur, v_prev, upd_mask, since_refresh, gave_up)
    if q_cur.shape != q_prev.shape or q_cur.stride() != q_prev.stride():
        raise ValueError("q_cur and q_prev must share shape and strides")
    g = GateDesc()
    g.mode = mode
    g.dtype = _dtype(q_cur)
    b, n, hq, d = q_cur.shape
    g.n_seq, g.n_blk, g.hq, g.d = b, n, hq, d
    if q_cur.stride(-1) != 1:
        raise ValueError("the head-dim axis must be contiguous")
    for i in range(3):
        g.q_stride[i] = q_cur.stride(i)
    g.q_cur, g.q_prev = q_cur.data_ptr(), q_prev.data_ptr()
    kv = k_cur if k_cur is not None else v_cur
    if kv is not None:
        for t in (k_cur, k_prev, v_cur, v_prev):
            if t is not None and (t.shape != kv.shape or t.stride() != kv.stride() or t.dtype != q_cur.dtype):
                raise ValueError("k/v tensors must share shape, strides and dtype")
        g.hkv = kv.shape[2]
        for i in range(3):
            g.kv_stride[i] = kv.stride(i)
    else:
        g.hkv = hq
    g.k_cur, g.k_prev, g.v_cur, g.v_prev = _ptr(k_cur), _ptr(k_prev), _ptr(v_cur), _ptr(v_prev)
    g.upd_mask = _ptr(upd_mask)
    g.tau = int(tau)
    g.gamma = float(gamma)
    g.cache_valid = 1 if cache_valid else 0
    if since_refresh is not None:
        _check_out(since_refresh, (g.n_seq, g.n_blk), torch.uint8, "since_refresh")
    g.since_refresh = _ptr(since_refresh)
    g.wait_polls = int(wait_polls)
    if gave_up is not None:
        _check_out(gave_up, (1,), torch.int32, "gave_up")
    g.gave_up = _ptr(gave_up)
    return g


def ba_reuse_gate_workspace(mode, q_cur, q_prev, **kw) -> int:
    g = _gate_desc(mode, q_cur, q_prev, kw.get("k_cur"), kw.get("k_prev"), kw.get("v_cur"),
                   kw.get("v_prev"), kw.get("upd_mask"), kw.get("tau", 0), kw.get("gamma", 0.0), True)
    return int(lib().ba_reuse_gate_workspace(ctypes.byref(g)))


def ba_reuse_gate(mode, q_cur, q_prev, *, decision, workspace, k_cur=None, k_prev=None, v_cur=None,
                  v_prev=None, upd_mask=None, tau=0, gamma=0.0, cache_valid=True, m_count=None,
                  cos=None, since_refresh=None, stream=None):
    """Reuse decisions (uint8 [n_seq, hq], 1 = reuse) from the count, cosine or cumulative
    count gate (the latter keeps its state in since_refresh, uint8 [n_seq, n_blk]); in rows mode
    decision is uint8 [n_seq, n_blk], 1 = the row's cached prefix part is current.
    `workspace` must be zero-filled before its first use (the call leaves it zeroed)."""
    g = _gate_desc(mode, q_cur, q_prev, k_cur, k_prev, v_cur, v_prev, upd_mask, tau, gamma, cache_valid,
                   since_refresh)
    _need_gpu(decision, workspace, m_count, cos)
    _check_out(decision, (g.n_seq, g.n_blk if mode == BA_GATE_ROWS else g.hq), torch.uint8, "decision")
    _check_out(m_count, (g.n_seq,), torch.int32, "m_count")
    _check_out(cos, (g.n_seq, g.hq), torch.float64, "cos")
    nbytes = workspace.numel() * workspace.element_size()
    check(lib().ba_reuse_gate(ctypes.byref(g), _ptr(m_count), _ptr(cos), _ptr(decision), _ptr(workspace),
                              nbytes, _stream(stream)))


def ba_gated_split_attn_gate_workspace(mode, q_cur, q_prev, **kw) -> int:
    g = _gate_desc(mode, q_cur, q_prev, kw.get("k_cur"), kw.get("k_prev"), kw.get("v_cur"),
                   kw.get("v_prev"), kw.get("upd_mask"), kw.get("tau", 0), kw.get("gamma", 0.0), True)
    return int(lib().ba_gated_split_attn_gate_workspace(ctypes.byref(g)))


def ba_gated_split_attn(mode, q_prev, kp, vp, k, v, a_out, l_out, a_in, l_in, a_full, l_full=None,
                        workspace=None, *, q, decision, gate_workspace, k_prev=None, v_prev=None,
                        upd_mask=None, tau=0, gamma=0.0, cache_valid=True, m_count=None, cos=None,
                        since_refresh=None, kv_layout="bhsd", scale=None, wait_polls=0, gave_up=None,
                        stream=None):
    """The reuse gate (q/k/v against q_prev/k_prev/v_prev; count or cosine mode) and the
    split attention it gates, as ba_reuse_gate followed by ba_split_attn with
    decision = (decision if cache_valid else None), in two launches.  Dense
    block tensors [B, Nb, H, d]; `gate_workspace` is sized by
    ba_gated_split_attn_gate_workspace and zero-filled before its first use.
    wait_polls bounds the prefix workgroups' wait for the gate (0 = default,
    < 0 = give up at once); gave_up (int32 [1]) counts the waits that gave up."""
    count = mode in (BA_GATE_COUNT, BA_GATE_COUNT_CUM)
    g = _gate_desc(mode, q, q_prev, k if count else None, k_prev if count else None,
                   v if count else None, v_prev if count else None, upd_mask, tau, gamma, cache_valid,
                   since_refresh, wait_polls, gave_up)
    _need_gpu(decision, gate_workspace, m_count, cos)
    _check_out(decision, (g.n_seq, g.hq), torch.uint8, "decision")
    _check_out(m_count, (g.n_seq,), torch.int32, "m_count")
    _check_out(cos, (g.n_seq, g.hq), torch.float64, "cos")
    dp, rows = _desc(q, kp, vp, q_layout="bshd", kv_layout=kv_layout, cu_q=None, cu_k=None,
                     max_q=None, max_k=None, scale=scale, decision=None)
    db, _ = _desc(q, k, v, q_layout="bshd", kv_layout="bshd", cu_q=None, cu_k=None,
                  max_q=None, max_k=None, scale=scale, decision=None)
    for t, nm in ((a_out, "a_out"), (a_in, "a_in"), (a_full, "a_full")):
        _check_out(t, (rows, dp.hq, dp.d), torch.float32, nm)
    for t, nm in ((l_out, "l_out"), (l_in, "l_in")):
        _check_out(t, (rows, dp.hq), torch.float32, nm)
    if l_full is not None:
        _check_out(l_full, (rows, dp.hq), torch.float32, "l_full")
    _need_gpu(workspace)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    gbytes = gate_workspace.numel() * gate_workspace.element_size()
    check(lib().ba_gated_split_attn(ctypes.byref(g), _ptr(m_count), _ptr(cos), _ptr(decision),
                                    _ptr(gate_workspace), gbytes, ctypes.byref(dp), ctypes.byref(db),
                                    _ptr(a_out), _ptr(l_out), _ptr(a_in), _ptr(l_in), _ptr(a_full),
                                    _ptr(l_full), _ptr(workspace), nbytes, _stream(stream)))


def ba_kl_lock(logits_cur, logits_prev, *, eps, kl=None, locked=None, eligible=None, stream=None):
    """KL(softmax(cur) || softmax(prev)) per row of [n, vocab] logits into kl (float32 [n]);
    rows with eligible != 0 (all if None) and KL < eps set locked (uint8 [n]) to 1."""
    _need_gpu(logits_cur, logits_prev, kl, locked, eligible)
    if logits_cur.shape != logits_prev.shape or logits_cur.dim() != 2 or logits_cur.dtype != logits_prev.dtype:
        raise ValueError("logits_cur and logits_prev must be [n, vocab] tensors of one dtype")
    if logits_cur.stride(1) != 1 or logits_prev.stride(1) != 1 or logits_cur.stride(0) != logits_prev.stride(0):
        raise ValueError("logit rows must be contiguous with one row stride")
    n, vocab = logits_cur.shape
    _check_out(kl, (n,), torch.float32, "kl")
    _check_out(locked, (n,), torch.uint8, "locked")
    _check_out(eligible, (n,), torch.uint8, "eligible")
    check(lib().ba_kl_lock(n, vocab, _dtype(logits_cur), _ptr(logits_cur), _ptr(logits_prev), logits_cur.stride(0),
                           _ptr(eligible), float(eps), _ptr(kl), _ptr(locked), _stream(stream)))


def ba_varlen_pack(block_sizes, locked, cu_seqlens_q, gather_idx, total, q_src=None, q_packed=None,
                   stream=None):
    """Pack unlocked positions (branch-major, ascending); q_src [N, h, d] rows are
    gathered into q_packed [N, h, d] when both are given."""
    _need_gpu(locked, cu_seqlens_q, gather_idx, total, q_src, q_packed)
    bs = [int(x) for x in block_sizes]
    arr = (ctypes.c_int32 * max(1, len(bs)))(*bs)
    n = sum(bs)
    _check_out(cu_seqlens_q, (len(bs) + 1,), torch.int32, "cu_seqlens_q")
    _check_out(gather_idx, (n,), torch.int32, "gather_idx")
    _check_out(total, (1,), torch.int32, "total")
    if locked is not None and (locked.dtype != torch.uint8 or locked.numel() < n):
        raise ValueError("locked must be uint8 with one entry per block position")
    dtype, h, d, st = 0, 0, 0, None
    if q_src is not None:
        dtype = _dtype(q_src)
        _, h, d = q_src.shape
        if q_src.stride(-1) != 1:
            raise ValueError("the head-dim axis must be contiguous")
        st = c_i64x2(q_src.stride(0), q_src.stride(1))
        _check_out(q_packed, (n, h, d), q_src.dtype, "q_packed")
    check(lib().ba_varlen_pack(len(bs), arr, _ptr(locked), _ptr(cu_seqlens_q), _ptr(gather_idx),
                               _ptr(total), dtype, h, d, _ptr(q_src), st, _ptr(q_packed), _stream(stream)))
