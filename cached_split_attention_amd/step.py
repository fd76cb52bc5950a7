"""One denoising step of cached split attention, as library calls.

FlashBlock (gist.science/es/paper/2602.05305), section 2: each step runs the
reuse gate, recomputes the out-of-block part (A_out, L_out) only for the
(sequence, head) pairs the gate sends to recompute (the kernel itself skips
the others, reading the decision from device memory, so there is no
device-to-host synchronisation), computes the in-block part (A_in, L_in),
and merges the two.  One call does it all (ba_gated_split_attn): the gate,
the in-block part and the gated prefix part share one launch (the prefix
workgroups wait for their sequence's decisions; the in-block part needs
none), and the pass that combines the prefix's key splits also does the
merge, so a step is two launches on one stream.  The cache stays valid
until the next block starts.  This module only orders calls and owns
buffers; it computes nothing itself.

Gate variants: "count_cum" counts the positions updated since each
sequence's cache was last written (its marks live in a buffer here);
"partial" refreshes the cache row by row instead of reusing it: the rows
whose Q changed are found (ba_reuse_gate, rows mode), listed
(ba_varlen_pack) and recomputed into the cache (ba_prefix_attn_rows), then
the in-block part is merged with it (ba_block_attn), so every step's result
equals a full recompute.
"""

from __future__ import annotations

import torch

from .api import (BA_GATE_COUNT, BA_GATE_COSINE, BA_GATE_COUNT_CUM, BA_GATE_ROWS, ba_block_attn,
                  ba_gated_split_attn, ba_gated_split_attn_gate_workspace, ba_prefix_attn_rows,
                  ba_prefix_attn_workspace, ba_reuse_gate, ba_reuse_gate_workspace, ba_varlen_pack)

GATE_MODES = {"count": BA_GATE_COUNT, "cosine": BA_GATE_COSINE, "count_cum": BA_GATE_COUNT_CUM,
              "partial": BA_GATE_ROWS}


class CachedBlockAttention:
    """State for one block's denoising schedule (dense layout).

    kp, kv: prefix K/V [B, Hkv, Lp, d] ("bhsd") or [B, Lp, Hkv, d] ("bshd").
    Block tensors passed to step() are [B, Nb, H, d].
    gate: "count" (tau on the number of updated positions), "count_cum"
    (tau on the number updated since the cache was last written), "cosine"
    (gamma on the per-head cosine of Q against the previous step's) or
    "partial" (recompute exactly the rows whose Q changed).
    """

    def __init__(self, kp, vp, *, nb, hq, gate="count", tau=0, gamma=0.0, scale=None,
                 kv_layout="bhsd"):
        self.kp, self.vp = kp, vp
        self.kv_layout = kv_layout
        self.B = kp.shape[0]
        self.hq, self.nb, self.d = hq, nb, kp.shape[-1]
        if gate not in GATE_MODES:
            raise ValueError(f"unknown gate {gate!r}")
        self.mode = GATE_MODES[gate]
        self.tau, self.gamma, self.scale = tau, gamma, scale
        dev = kp.device
        rows = self.B * nb
        self.a_out = torch.zeros(rows, hq, self.d, device=dev, dtype=torch.float32)
        self.l_out = torch.zeros(rows, hq, device=dev, dtype=torch.float32)
        self.a_full = torch.empty(rows, hq, self.d, device=dev, dtype=torch.float32)
        self.l_full = torch.empty(rows, hq, device=dev, dtype=torch.float32)
        self.a_in = torch.empty(rows, hq, self.d, device=dev, dtype=torch.float32)
        self.l_in = torch.empty(rows, hq, device=dev, dtype=torch.float32)
        self.decision = torch.zeros(self.B, hq, device=dev, dtype=torch.uint8)
        self.m_count = torch.zeros(self.B, device=dev, dtype=torch.int32)
        self.cos = torch.zeros(self.B, hq, device=dev, dtype=torch.float64)
        # prefix workgroups whose bounded wait for their gate gave up (the
        # result does not depend on it; a nonzero count means the gate ran
        # far slower than expected)
        self.gave_up = torch.zeros(1, device=dev, dtype=torch.int32)
        if self.mode == BA_GATE_COUNT_CUM:
            self.since_refresh = torch.zeros(self.B, nb, device=dev, dtype=torch.uint8)
        if self.mode == BA_GATE_ROWS:
            # per-row "cache is current" marks, then the list of rows to redo
            self.decision = torch.zeros(self.B, nb, device=dev, dtype=torch.uint8)
            self.cu_rows = torch.zeros(self.B + 1, device=dev, dtype=torch.int32)
            self.rows = torch.zeros(max(rows, 1), device=dev, dtype=torch.int32)
            self.n_rows = torch.zeros(1, device=dev, dtype=torch.int32)
        self.cache_valid = False
        self._ws = None
        self._gws = None

    def start_block(self, kp=None, vp=None):
        """Invalidate the cache (a new block begins; the prefix may have grown)."""
        if kp is not None:
            if kp.shape != self.kp.shape:
                self._ws = None
            self.kp, self.vp = kp, vp
        self.cache_valid = False

    def _workspaces(self, q, k, v, q_prev, k_prev, v_prev):
        if self._ws is None:
            n = ba_prefix_attn_workspace(q, self.kp, self.vp, kv_layout=self.kv_layout, scale=self.scale)
            self._ws = torch.zeros(max(n, 1), device=q.device, dtype=torch.uint8)
        if self._gws is None:
            if self.mode == BA_GATE_ROWS:
                n = ba_reuse_gate_workspace(self.mode, q, q_prev)
            else:
                kw = {} if self.mode == BA_GATE_COSINE else dict(k_cur=k, k_prev=k_prev, v_cur=v, v_prev=v_prev)
                n = ba_gated_split_attn_gate_workspace(self.mode, q, q_prev, **kw)
            self._gws = torch.zeros(max(n, 1), device=q.device, dtype=torch.uint8)

    def step(self, q, k, v, q_prev, k_prev, v_prev, stream=None, upd_mask=None):
        """Run one step; returns (a_full, l_full) views of the output buffers.

        With no valid cache the gate still runs (it reports M), but the prefix
        part is not gated by it: everything recomputes.  upd_mask (uint8
        [B, Nb], count gates only): the caller's own record of the positions it
        updated since the previous step, counted instead of comparing rows."""
        if upd_mask is not None and self.mode not in (BA_GATE_COUNT, BA_GATE_COUNT_CUM):
            raise ValueError("an update mask feeds the count gates only")
        self._workspaces(q, k, v, q_prev, k_prev, v_prev)
        main = stream if stream is not None else torch.cuda.current_stream()
        if self.mode == BA_GATE_ROWS:
            self._partial_step(q, k, v, q_prev, main)
            self.cache_valid = True
            return self.a_full, self.l_full
        count = self.mode in (BA_GATE_COUNT, BA_GATE_COUNT_CUM)
        ba_gated_split_attn(self.mode, q_prev, self.kp, self.vp, k, v, self.a_out, self.l_out, self.a_in,
                            self.l_in, self.a_full, self.l_full, self._ws, q=q, decision=self.decision,
                            gate_workspace=self._gws, k_prev=k_prev if count else None,
                            v_prev=v_prev if count else None, upd_mask=upd_mask, tau=self.tau, gamma=self.gamma,
                            cache_valid=self.cache_valid, m_count=self.m_count if count else None,
                            cos=None if count else self.cos,
                            since_refresh=getattr(self, "since_refresh", None), kv_layout=self.kv_layout,
                            scale=self.scale, gave_up=self.gave_up, stream=main)
        self.cache_valid = True
        return self.a_full, self.l_full

    def waits_given_up(self) -> int:
        """Prefix workgroups that gave up waiting for their gate so far (reads
        the device counter; synchronises)."""
        return int(self.gave_up.item())

    def _partial_step(self, q, k, v, q_prev, stream):
        # rows whose Q is unchanged keep their cached prefix part (all rows
        # are redone when there is no cache yet)
        ba_reuse_gate(BA_GATE_ROWS, q, q_prev, decision=self.decision, workspace=self._gws,
                      cache_valid=self.cache_valid, m_count=self.m_count, stream=stream)
        ba_varlen_pack([self.nb] * self.B, self.decision.view(-1), self.cu_rows, self.rows[:self.B * self.nb],
                       self.n_rows, stream=stream)
        ba_prefix_attn_rows(q, self.kp, self.vp, self.cu_rows, self.rows[:self.B * self.nb], self.a_out,
                            self.l_out, self._ws, kv_layout=self.kv_layout, scale=self.scale, stream=stream)
        ba_block_attn(q, k, v, a_cache=self.a_out, l_cache=self.l_out, a_in=self.a_in, l_in=self.l_in,
                      a_full=self.a_full, l_full=self.l_full, scale=self.scale, stream=stream)

    def capture(self, q, k, v, steps, new_block=True, kp=None, vp=None, masks=None):
        """Capture the given steps of a block's schedule as one HIP graph.

        q, k, v: sequences of block tensors, index 0 = the block before step 1,
        index t = the block at step t.  With new_block the graph starts a new
        block (no valid cache); otherwise the cache is taken as valid.
        Replaying the graph re-runs those steps on the same buffers.
        masks: optional per-step update masks (masks[t] for step t), as in step().
        Workspaces are allocated before capture and no memset is recorded
        (the gate's tickets are cleared by its own workgroups and its ready
        counts by the combine pass), so replays need no re-initialisation.
        """
        steps = list(steps)
        self.start_block(kp, vp)
        t0 = steps[0]
        self._workspaces(q[t0], k[t0], v[t0], q[t0 - 1], k[t0 - 1], v[t0 - 1])
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                self.cache_valid = not new_block
                for t in steps:
                    self.step(q[t], k[t], v[t], q[t - 1], k[t - 1], v[t - 1],
                              stream=torch.cuda.current_stream(),
                              upd_mask=None if masks is None else masks[t])
        torch.cuda.current_stream().wait_stream(side)
        self.cache_valid = True
        return graph

    def capture_block(self, q, k, v, kp=None, vp=None, masks=None):
        """One block's whole schedule (steps 1 .. len(q)-1) as one graph."""
        return self.capture(q, k, v, range(1, len(q)), new_block=True, kp=kp, vp=vp, masks=masks)
