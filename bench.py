#!/usr/bin/env python3
"""Benchmark of cached split attention for block diffusion on one MI355X.

Default workload: the long-context grouped-query shape (batch 8, 32 query
heads sharing 8 KV heads, head dim 128, bf16, prefix 32768, block 64, 64
denoising steps per block, Poisson(3) rewritten block rows per step, count
gate with tau = 8): the largest of the workload shapes.  One bench step is
one block's whole schedule: for every denoising step the reuse gate, the
gate-predicated prefix (out-of-block) pass, and the in-block pass with the
fused log-space merge.  The first denoising step of a block has no valid
cache and recomputes the prefix part.  Inputs are seeded synthetic tensors,
resident in HBM before timing starts; the prefix K/V is rotated over copies
totalling at least 1 GiB so a recompute reads it from HBM, not from the
256 MB last-level cache.

Prints one JSON line.  value = algorithmic bytes moved per second (GB/s);
TFLOP/s, per-step latencies, the prefix kernel's roofline, the in-block
part's rate and the CPU oracle's rate on a bounded sample ride along.
--workload selects another of the workload shapes (c2_llada: the LLaDA-like
heads; c4_video; c1_tiny_f32); the multi-branch varlen one (c5_varlen) times
one step with a cold cache (varlen packing, then the split attention);
kl_lock times the lock criterion; --lp and --sparse give the long-context
and sparse residual-reuse legs of the dense shapes.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-attn step TFLOP/s + KV GB/s (% of MI355X roofline); per-step latency"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
KERNEL_SOURCES = ["cached_split_attention_amd/csrc/attn_bf16.hip"]
KL_SOURCES = ["cached_split_attention_amd/csrc/kl.hip"]


# ----------------------------------------------------------------------------
# algorithmic work (what the method itself reads, writes and computes)
# ----------------------------------------------------------------------------

def step_work(s, dec, esize=2, mask=False):
    """Algorithmic (bytes, flops, prefix_bytes, prefix_flops) of one
    denoising step of schedule s with decision matrix dec [B, Hq] (1 = reuse),
    or, for the partial refresh, per-row marks dec [B, Nb] (1 = row current).
    Prefix: K/V of every KV head with a recomputed query head (partial: of
    every sequence with a recomputed row), the recomputed Q rows, their
    A_out/L_out written.  Every step: gate inputs (the update mask, with
    mask), block Q, K, V, the cache
    read by the merge, A_full/L_full written."""
    B, hq, hkv, d, lp, nb = s.B, s.hq, s.hkv, s.d, s.lp, s.nb
    g = hq // hkv
    rec = (dec == 0)
    if s.gate == "partial":
        n_rows = int(rec.sum())
        seqs = int(rec.any(axis=1).sum())
        p_bytes = seqs * hkv * lp * d * esize * 2 + n_rows * hq * d * esize + n_rows * hq * (d + 1) * 4
        p_flops = 4 * d * lp * n_rows * hq
    else:
        n_rec = int(rec.sum())
        kv_heads = int(rec.reshape(B, hkv, g).any(axis=2).sum())
        p_bytes = kv_heads * lp * d * esize * 2 + n_rec * nb * d * esize + n_rec * nb * (d + 1) * 4
        p_flops = 4 * d * nb * lp * n_rec
    if s.gate in ("count", "count_cum") and mask:
        gate_bytes = B * nb   # the caller's update mask
    elif s.gate in ("count", "count_cum"):
        gate_bytes = 2 * B * nb * (hq + 2 * hkv) * d * esize
    else:
        gate_bytes = 2 * B * nb * hq * d * esize
    blk_bytes = (B * nb * hq * d * esize + 2 * B * nb * hkv * d * esize
                 + 2 * B * nb * hq * (d + 1) * 4)
    blk_flops = 4 * d * nb * nb * B * hq
    return p_bytes + gate_bytes + blk_bytes, p_flops + blk_flops, p_bytes, p_flops


def varlen_work(vb, total):
    """Algorithmic (bytes, flops, prefix_bytes, prefix_flops) of one step of
    the multi-branch varlen batch vb with a cold cache and `total` unlocked
    (packed) query rows: the lock mask read and the packing indices written,
    the unlocked Q rows gathered (read and written), every branch's prefix
    K/V, the packed Q read by the attention, A_out/L_out written and read by
    the merge, the block K/V, A_full/L_full written."""
    import numpy as np
    H, d, es = vb.h, vb.d, 2
    bs = vb.block_sizes.astype(np.int64)
    ltot, btot, nbr = int(vb.prefix_lens.sum()), int(bs.sum()), int(bs.size)
    pack = btot + (nbr + 1) * 4 + btot * 4 + 4 + 2 * total * H * d * es
    p_bytes = 2 * ltot * H * d * es + total * H * d * es + total * H * (d + 1) * 4
    blk_bytes = 2 * btot * H * d * es + total * H * (d + 1) * 4 + total * H * (d + 1) * 4
    starts = np.concatenate([[0], np.cumsum(bs)])
    u = np.array([int((vb.locked[starts[b]:starts[b + 1]] == 0).sum()) for b in range(nbr)], dtype=np.int64)
    p_flops = int(4 * d * H * (u * vb.prefix_lens.astype(np.int64)).sum())
    blk_flops = int(4 * d * H * (u * bs).sum())
    return pack + p_bytes + blk_bytes, p_flops + blk_flops, p_bytes, p_flops


# ----------------------------------------------------------------------------
# measured HBM traffic of the prefix kernel (rocprofv3 counters), if current
# ----------------------------------------------------------------------------

def kernel_source_hash(sources=KERNEL_SOURCES):
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, name=None, sources=KERNEL_SOURCES):
    """Per-launch HBM bytes of the prefix kernel (or of the kernel whose
    summary is profiles/<name>_traffic.md) from the committed counter
    summary, or None if absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"{name or 'prefix_attn_' + workload}_traffic.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256_16") != kernel_source_hash(sources):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ----------------------------------------------------------------------------
# CPU baseline: the oracle, as it stands, on a bounded sample
# ----------------------------------------------------------------------------

def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def host_cores():
    """Cores this process may run on, the BLAS thread count and the CPU model."""
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    model = None
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
    except Exception:  # noqa: BLE001
        pass
    return {"affinity_cores": affinity, "blas_threads": int(threads), "cpu_model": model or cpu_model()}


def cpu_baseline(s, budget_s=12.0, got=None):
    """The oracle, as it stands, on a bounded sample of the workload: whole
    block schedules of one (sequence, query head) after another -- the gate
    over the block, then per step the prefix part when that head recomputes,
    the in-block part and the merge -- until budget_s has passed.  The rate
    is the schedule's algorithmic bytes scaled to the pairs done.  When the
    GPU's final-step A_full/L_full are given, the errors the GPU path
    achieves on the sampled pairs are reported too."""
    import numpy as np
    import oracle
    cores = host_cores()
    t0 = time.perf_counter()
    gates = oracle.step_gates(s)
    pairs = [(b, h) for b in range(s.B) for h in range(s.hq)]
    done = []
    finals = {}
    for b, h in pairs:
        ao = lo = None
        for t in range(1, s.steps + 1):
            if ao is None or gates[t]["decision"][b, h] == 0:
                ao, lo = oracle.prefix_rows(s, t, b, h)
            ai, li = oracle.block_rows(s, t, b, h)
            af, lf = oracle.merge(ao, lo, ai, li)
        finals[(b, h)] = (af, lf)
        done.append((b, h))
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    sched_bytes = sum(step_work(s, gates[t]["decision"])[0] for t in range(1, s.steps + 1))
    frac = len(done) / len(pairs)
    out = {"value": sched_bytes * frac / dt / 1e9, "unit": "GB/s", "cores": cores["blas_threads"],
           "kind": "oracle",
           "sample": f"the whole {s.steps}-step block schedule (gate, prefix part on recomputing steps, "
                     f"in-block part, merge) of {len(done)} of {len(pairs)} (sequence, query head) pairs, "
                     f"bytes scaled to those pairs, NumPy float64, {dt:.1f} s",
           "ms_per_step": dt / frac / s.steps * 1e3, **cores}
    if got is not None:
        ga, gl = got
        ga = ga.reshape(s.B, s.nb, s.hq, s.d)
        gl = gl.reshape(s.B, s.nb, s.hq)
        wa = np.stack([finals[p][0] for p in done])
        wl = np.stack([finals[p][1] for p in done])
        pa = np.stack([ga[b, :, h] for b, h in done])
        pl = np.stack([gl[b, :, h] for b, h in done])
        out["achieved_error"] = {
            "step": s.steps, "rows": int(len(done) * s.nb),
            "a_full_max_abs": float(np.abs(pa - wa).max()),
            "a_full_rel_l2": float(np.linalg.norm(pa - wa) / np.linalg.norm(wa)),
            "l_full_max_abs": float(np.abs(pl - wl).max()),
            "bars": {"a_max_abs": 2e-2, "a_rel_l2": 5e-3, "l_max_abs": 1e-4}}
    return out


# ----------------------------------------------------------------------------
# GPU run
# ----------------------------------------------------------------------------

COPY_PROBE_BYTES = 256 << 20
REUSE_REPS = 16   # reuse steps per graph in the reuse-step latency leg


def measured_peaks(dev):
    """A peak measured on this machine, outside any timed region: a device copy
    of 1 GiB (bytes read + written per second).  Context only: the roofline
    fractions are against the published peaks."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    n = (1 << 30) // 4
    src = torch.ones(n, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(5):
        dst.copy_(src)
    ev[1].record()
    torch.cuda.synchronize()
    copy_gbs = 2 * 5 * n * 4 / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e9
    del src, dst
    return {"copy_gbs": round(copy_gbs, 1)}


def with_measured(roof, peaks):
    """The roofline block plus the measured copy rate (context)."""
    return {**roof, "measured_peak": peaks}


def probe(args, s, q, kps, vps):
    """Launches for per-dispatch counter collection: 2 passes over the
    rotated prefix copies (every head recomputes), then 4 device-to-device
    copies of COPY_PROBE_BYTES, whose counter readings calibrate the bytes
    per counter unit."""
    import torch
    import cached_split_attention_amd as ba
    dev = q[1].device
    ws = torch.zeros(max(1, ba.ba_prefix_attn_workspace(q[1], kps[0], vps[0], scale=s.scale)), device=dev,
                     dtype=torch.uint8)
    rows = s.B * s.nb
    a = torch.empty(rows, s.hq, s.d, device=dev)
    l = torch.empty(rows, s.hq, device=dev)
    for i in range(2 * len(kps)):
        ba.ba_prefix_attn(q[1], kps[i % len(kps)], vps[i % len(kps)], a, l, ws, scale=s.scale)
    torch.cuda.synchronize()
    src = torch.ones(COPY_PROBE_BYTES // 4, device=dev)
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"probe": args.workload, "prefix_passes": 2 * len(kps),
                      "copy_bytes_each": COPY_PROBE_BYTES, "copies": 4}), flush=True)

def probe_inblock(args, s, q, k, v, kps, vps):
    """Launches for per-dispatch counters of the in-block part alone: the
    cache is filled by one prefix pass, then 4 ba_block_attn calls over the
    last step's block with the fused merge (A_in/L_in and A_full/L_full
    written), eagerly."""
    import torch
    import cached_split_attention_amd as ba
    dev = q[1].device
    ws = torch.zeros(max(1, ba.ba_prefix_attn_workspace(q[1], kps[0], vps[0], scale=s.scale)), device=dev,
                     dtype=torch.uint8)
    rows = s.B * s.nb
    a_out = torch.empty(rows, s.hq, s.d, device=dev)
    l_out = torch.empty(rows, s.hq, device=dev)
    ba.ba_prefix_attn(q[s.steps], kps[0], vps[0], a_out, l_out, ws, scale=s.scale)
    outs = [torch.empty_like(a_out), torch.empty_like(l_out), torch.empty_like(a_out), torch.empty_like(l_out)]
    torch.cuda.synchronize()
    for _ in range(4):
        ba.ba_block_attn(q[s.steps], k[s.steps], v[s.steps], a_cache=a_out, l_cache=l_out, a_in=outs[0],
                         l_in=outs[1], a_full=outs[2], l_full=outs[3], scale=s.scale)
    torch.cuda.synchronize()
    print(json.dumps({"probe_inblock": args.workload, "calls": 4,
                      "algorithmic_flops_per_call": 4 * s.d * s.nb * s.nb * s.B * s.hq}), flush=True)


def roofline_of(p_bytes, p_flops, us):
    """The roof a pass of this arithmetic intensity reaches first, and the
    fraction of it achieved in `us` microseconds."""
    achieved = p_bytes / (us * 1e-6) / 1e9
    achieved_tf = p_flops / (us * 1e-6) / 1e12
    if p_flops / p_bytes > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": round(achieved_tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved_tf / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    return roof, achieved, achieved_tf


def run_varlen(args):
    """The multi-branch varlen workload: one step with a cold cache = the
    packing of unlocked positions, then the split attention (prefix and
    in-block parts in one launch, then combine and merge), captured as one
    HIP graph per rotated prefix copy."""
    import numpy as np
    import torch
    import cached_split_attention_amd as ba
    from workloads import preset

    dev = torch.device("cuda:0")
    vb = preset(args.workload)

    def to_dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)

    n = int(vb.block_sizes.sum())
    nbr = int(vb.block_sizes.size)
    kp0, vp0 = to_dev(vb.kp), to_dev(vb.vp)
    kv_bytes = 2 * kp0.numel() * 2
    n_copies = max(1, int(math.ceil(args.cold_bytes * (1 << 30) / kv_bytes)))
    kps = [kp0] + [kp0.clone() for _ in range(n_copies - 1)]
    vps = [vp0] + [vp0.clone() for _ in range(n_copies - 1)]
    q_all, kb, vbk = to_dev(vb.q), to_dev(vb.k), to_dev(vb.v)
    locked = torch.from_numpy(vb.locked).to(dev)
    cu_q = torch.empty(nbr + 1, device=dev, dtype=torch.int32)
    gather = torch.empty(n, device=dev, dtype=torch.int32)
    total = torch.empty(1, device=dev, dtype=torch.int32)
    qp = torch.zeros(n, vb.h, vb.d, device=dev, dtype=torch.bfloat16)
    cu_kp = torch.from_numpy(np.concatenate([[0], np.cumsum(vb.prefix_lens)]).astype(np.int32)).to(dev)
    cu_kb = torch.from_numpy(np.concatenate([[0], np.cumsum(vb.block_sizes)]).astype(np.int32)).to(dev)
    max_q, max_kp, max_kb = int(vb.block_sizes.max()), int(vb.prefix_lens.max()), int(vb.block_sizes.max())
    outs = {nm: torch.empty(n, vb.h, vb.d, device=dev) for nm in ("a_out", "a_in", "a_full")}
    outs.update({nm: torch.empty(n, vb.h, device=dev) for nm in ("l_out", "l_in", "l_full")})
    pkw = dict(q_layout="thd", kv_layout="htd", cu_q=cu_q, cu_k=cu_kp, max_q=max_q, max_k=max_kp,
               scale=vb.scale)
    ws = torch.zeros(max(1, ba.ba_prefix_attn_workspace(qp, kp0, vp0, **pkw)), device=dev, dtype=torch.uint8)

    def step(i, stream=None):
        ba.ba_varlen_pack(vb.block_sizes, locked, cu_q, gather, total, q_all, qp, stream=stream)
        ba.ba_split_attn(qp, kps[i], vps[i], kb, vbk, outs["a_out"], outs["l_out"], outs["a_in"], outs["l_in"],
                         outs["a_full"], outs["l_full"], ws, q_layout="thd", kv_layout="htd",
                         block_kv_layout="thd", cu_q=cu_q, cu_kp=cu_kp, cu_k=cu_kb, max_q=max_q,
                         max_kp=max_kp, max_k=max_kb, scale=vb.scale, stream=stream)

    def prefix_pass(i, stream=None):
        ba.ba_prefix_attn(qp, kps[i], vps[i], outs["a_out"], outs["l_out"], ws, stream=stream, **pkw)

    step(0)
    torch.cuda.synchronize()
    n_total = int(total.item())
    if args.probe:
        for i in range(2 * n_copies):
            prefix_pass(i % n_copies)
        torch.cuda.synchronize()
        src = torch.ones(COPY_PROBE_BYTES // 4, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"probe": args.workload, "prefix_passes": 2 * n_copies,
                          "copy_bytes_each": COPY_PROBE_BYTES, "copies": 4}), flush=True)
        return
    stream = torch.cuda.current_stream()

    def capture(fn, i):
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                fn(i, stream=torch.cuda.current_stream())
        stream.wait_stream(side)
        return g

    graphs = [capture(step, i) for i in range(n_copies)]
    pgraphs = [capture(prefix_pass, i) for i in range(n_copies)]

    def timed(fn, n_rep):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n_rep):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n_rep

    for i in range(args.warmup):
        graphs[i % n_copies].replay()
    torch.cuda.synchronize()
    K = args.steps
    w0 = time.perf_counter()
    ms_per_step = timed(lambda i: graphs[(args.warmup + i) % n_copies].replay(), K)
    wall = time.perf_counter() - w0
    pref_us = timed(lambda i: pgraphs[i % n_copies].replay(), max(4, 2 * n_copies)) * 1e3

    s_bytes, s_flops, p_bytes, p_flops = varlen_work(vb, n_total)
    roof, achieved, achieved_tf = roofline_of(p_bytes, p_flops, pref_us)
    if not args.no_peaks:
        roof = with_measured(roof, measured_peaks(dev))
    out = {
        "metric": METRIC,
        "value": round(s_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic, seeded (workloads.preset), resident in HBM",
        "config": {"workload": f"{args.workload}: branches with block sizes {vb.block_sizes.tolist()}, "
                               f"prefixes {vb.prefix_lens.tolist()}, H={vb.h} d={vb.d}, "
                               f"{n_total} unlocked of {n} positions",
                   "bench_step": "one step with a cold cache (varlen pack, then split attention), "
                                 "replayed as a HIP graph",
                   "prefix_kv_copies": n_copies},
        "tflops": round(s_flops / (ms_per_step * 1e-3) / 1e12, 4),
        "latency_us": {"step": round(ms_per_step * 1e3, 2), "prefix_pass": round(pref_us, 2)},
        "roofline": {
            "kernel": "prefix pass (varlen, every branch): split-KV attention kernel + split combine kernel, "
                      "back to back",
            **roof,
            "traffic": measured_traffic(args.workload),
            "algorithmic_bytes_per_launch": p_bytes,
            "algorithmic_flops_per_launch": p_flops,
            "gbs": round(achieved, 1),
            "tflops": round(achieved_tf, 3),
        },
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        import oracle
        cores = host_cores()
        heads = list(range(0, vb.h, 4))
        t0 = time.perf_counter()
        oracle.run_varlen(vb, heads=heads)
        dt = time.perf_counter() - t0
        frac = len(heads) / vb.h
        out["cpu_baseline"] = {"value": s_bytes * frac / dt / 1e9, "unit": "GB/s",
                               "cores": cores["blas_threads"], **cores, "kind": "oracle",
                               "sample": f"one step of the same batch on {len(heads)} of {vb.h} heads "
                                         f"(bytes scaled to those heads), NumPy float64, {dt:.1f} s"}
    print(json.dumps(out), flush=True)


def run_sparse(args, s, q, kps, vps):
    """Sparse-attention residual reuse on a dense shape: each step attends
    fresh over a key-block selection (density args.sparse) and merges the
    result with the cached residual over the unselected blocks (computed
    once, at a refresh).  Times the selected pass plus the merge (the
    steady-state prefix part of a step), the residual pass (the refresh) and
    the dense pass, all with every head recomputing and the prefix copies
    rotated."""
    import numpy as np
    import torch
    import cached_split_attention_amd as ba
    from workloads import make_key_block_lists
    dev = q[1].device
    sel, rest = make_key_block_lists(B=s.B, hkv=s.hkv, lp=s.lp, density=args.sparse, seed=s.seed + 100)
    bsel = torch.from_numpy(sel).to(dev)
    brest = torch.from_numpy(rest).to(dev)
    rows = s.B * s.nb
    n_copies = len(kps)
    bufs = {nm: torch.empty(rows, s.hq, s.d, device=dev) for nm in ("a_sel", "a_res", "a_out", "a_dense")}
    bufs.update({nm: torch.empty(rows, s.hq, device=dev) for nm in ("l_sel", "l_res", "l_out", "l_dense")})
    ws_s = torch.zeros(max(1, ba.ba_sparse_prefix_attn_workspace(q[1], kps[0], vps[0], bsel, scale=s.scale)),
                       device=dev, dtype=torch.uint8)
    ws_r = torch.zeros(max(1, ba.ba_sparse_prefix_attn_workspace(q[1], kps[0], vps[0], brest, scale=s.scale)),
                       device=dev, dtype=torch.uint8)
    ws_d = torch.zeros(max(1, ba.ba_prefix_attn_workspace(q[1], kps[0], vps[0], scale=s.scale)), device=dev,
                       dtype=torch.uint8)
    stream = torch.cuda.current_stream()

    def sparse_step(i, st):
        ba.ba_sparse_prefix_attn(q[1], kps[i], vps[i], bsel, bufs["a_sel"], bufs["l_sel"], ws_s, scale=s.scale,
                                 stream=st)
        ba.ba_lse_merge(bufs["a_sel"], bufs["l_sel"], bufs["a_res"], bufs["l_res"], bufs["a_out"], bufs["l_out"],
                        stream=st)

    def residual(i, st):
        ba.ba_sparse_prefix_attn(q[1], kps[i], vps[i], brest, bufs["a_res"], bufs["l_res"], ws_r, scale=s.scale,
                                 stream=st)

    def dense(i, st):
        ba.ba_prefix_attn(q[1], kps[i], vps[i], bufs["a_dense"], bufs["l_dense"], ws_d, scale=s.scale, stream=st)

    def graph_of(fn):
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for i in range(n_copies):
                    fn(i, torch.cuda.current_stream())
        stream.wait_stream(side)
        return g

    residual(0, stream)
    sparse_step(0, stream)
    torch.cuda.synchronize()
    graphs = {nm: graph_of(fn) for nm, fn in (("sparse", sparse_step), ("residual", residual), ("dense", dense))}

    def timed(g, n_rep):
        g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n_rep):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (n_rep * n_copies)

    w0 = time.perf_counter()
    us = {nm: timed(g, args.steps if nm == "sparse" else 4) for nm, g in graphs.items()}
    wall = time.perf_counter() - w0
    # algorithmic bytes: the selected K/V, Q, the partial A/L written, the
    # cached residual read and A_out/L_out written by the merge
    es = 2
    ent = rows * s.hq
    n_blk = (s.lp + 63) // 64
    k_sel = int(sel.shape[2])
    # selected keys summed over (sequence, KV head): a ragged last block counts its own length
    kv_keys = sum(min(64 * (int(j) + 1), s.lp) - 64 * int(j) for j in sel.reshape(-1))
    sel_bytes = kv_keys * s.d * es * 2 + ent * s.d * es + ent * (s.d + 1) * 4
    step_bytes = sel_bytes + 2 * ent * (s.d + 1) * 4
    sel_flops = 4 * s.d * s.nb * kv_keys * (s.hq // s.hkv)
    roof, achieved, achieved_tf = roofline_of(sel_bytes, sel_flops, us["sparse"])
    out = {
        "metric": METRIC,
        "value": round(step_bytes / (us["sparse"] * 1e-6) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": 1,
        "ms_per_step": round(us["sparse"] * 1e-3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic, seeded (workloads.preset, make_key_block_lists), resident in HBM",
        "config": {"workload": f"{args.workload} with sparse prefix attention: B={s.B} Hq={s.hq} Hkv={s.hkv} "
                               f"d={s.d} prefix={s.lp}, {k_sel} of {n_blk} 64-key blocks selected per KV head "
                               f"(density {args.sparse})",
                   "bench_step": "the prefix part of a sparse step: the pass over the selected blocks, then the "
                                 "merge with the cached residual; every head recomputes",
                   "prefix_kv_copies": n_copies},
        "tflops": round(sel_flops / (us["sparse"] * 1e-6) / 1e12, 4),
        "latency_us": {"sparse_pass_and_merge": round(us["sparse"], 2), "residual_pass": round(us["residual"], 2),
                       "dense_pass": round(us["dense"], 2)},
        "roofline": {"kernel": "selected-block prefix pass + residual merge, back to back", **roof,
                     "traffic": None, "algorithmic_bytes_per_launch": int(sel_bytes),
                     "algorithmic_flops_per_launch": int(sel_flops), "gbs": round(achieved, 1),
                     "tflops": round(achieved_tf, 3)},
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        import oracle
        cores = host_cores()
        g = s.hq // s.hkv
        t0 = time.perf_counter()
        done = 0
        for h in range(s.hq):
            for b in range(s.B):
                a1, l1 = oracle.prefix_rows_in_blocks(s, 1, b, h, sel[b, h // g])
                done += 1
            if time.perf_counter() - t0 > 10.0:
                break
        dt = time.perf_counter() - t0
        frac = done / (s.B * s.hq)
        out["cpu_baseline"] = {"value": sel_bytes * frac / dt / 1e9, "unit": "GB/s",
                               "cores": cores["blas_threads"], **cores, "kind": "oracle",
                               "sample": f"the selected-block pass of {done} of {s.B * s.hq} (sequence, head) pairs, "
                                         f"bytes scaled to those, NumPy float64, {dt:.1f} s"}
    print(json.dumps(out), flush=True)


KL_ROWS, KL_VOCAB = 252, 126464   # the varlen batch's block positions; a vocabulary size chosen here


def run_yardstick(args, s, q, kps, vps):
    """Same-box yardstick: torch's fused attention (scaled_dot_product_attention,
    flash backend forced, so nothing falls back to unfused products) on the
    prefix-pass shape of this workload, next to the library's own prefix pass
    over the same rotated copies.  The query heads of one KV head are packed as
    one head of G*Nb rows, which is the same arithmetic; the output is checked
    against the library's A_out."""
    import torch
    import cached_split_attention_amd as ba
    from torch.nn.attention import SDPBackend, sdpa_kernel
    dev = q[1].device
    B, hq, hkv, d, nb = s.B, s.hq, s.hkv, s.d, s.nb
    g = hq // hkv
    qp = q[1].view(B, nb, hkv, g, d).permute(0, 2, 3, 1, 4).reshape(1, B * hkv, g * nb, d).contiguous()
    kq = [k.view(1, B * hkv, s.lp, d) for k in kps]
    vq = [v.view(1, B * hkv, s.lp, d) for v in vps]
    ws = torch.zeros(max(1, ba.ba_prefix_attn_workspace(q[1], kps[0], vps[0], scale=s.scale)), device=dev,
                     dtype=torch.uint8)
    a = torch.empty(B * nb, hq, d, device=dev)
    l = torch.empty(B * nb, hq, device=dev)
    n = max(6, 2 * len(kps))

    def timed(fn):
        # warm-up of about 0.3 s, so that the clocks have settled
        t_end = time.perf_counter() + 0.3
        while time.perf_counter() < t_end:
            for i in range(len(kps)):
                fn(i)
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            fn(i % len(kps))
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    out = {"yardstick": args.workload, "shape": {"heads": B * hkv, "rows": g * nb, "keys": s.lp, "d": d}}
    def ours_pass(i):
        ba.ba_prefix_attn(q[1], kps[i], vps[i], a, l, ws, scale=s.scale)

    ours_before = timed(ours_pass)
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            res = {}
            sd = timed(lambda i: res.__setitem__(0, torch.nn.functional.scaled_dot_product_attention(
                qp, kq[i], vq[i], scale=s.scale)))
            o = torch.nn.functional.scaled_dot_product_attention(qp, kq[0], vq[0], scale=s.scale)
        ours = (ours_before + timed(ours_pass)) / 2   # before and after, against clock drift
        out["ours_prefix_pass_us"] = round(ours, 2)
        ba.ba_prefix_attn(q[1], kps[0], vps[0], a, l, ws, scale=s.scale)
        mine = a.view(B, nb, hkv, g, d).permute(0, 2, 3, 1, 4).reshape(1, B * hkv, g * nb, d)
        torch.cuda.synchronize()
        out["torch_sdpa_flash_us"] = round(sd, 2)
        out["torch_rocm_fa_library"] = str(torch.backends.cuda.preferred_rocm_fa_library())
        out["speedup"] = round(sd / ours, 2)
        out["max_abs_diff_vs_a_out"] = float((o.float() - mine).abs().max().item())
        flops = 4.0 * d * nb * s.lp * hq * B
        out["tflops"] = {"ours": round(flops / ours / 1e6, 1), "torch_sdpa_flash": round(flops / sd / 1e6, 1)}
    except Exception as ex:   # no flash kernel for this shape or build
        out["ours_prefix_pass_us"] = round(ours_before, 2)
        out["torch_sdpa_flash_us"] = None
        out["error"] = f"{type(ex).__name__}: {str(ex)[:200]}"
    print(json.dumps(out), flush=True)


def run_kl(args):
    """The lock criterion on its own: KL of each token's posterior from the
    previous step's over a 126464-entry vocabulary, for the 252 block
    positions of the multi-branch varlen batch, bf16 logits, with the lock
    update; logit copies rotated over at least args.cold_bytes GiB so the
    rows come from HBM."""
    import numpy as np
    import torch
    import cached_split_attention_amd as ba
    from workloads import make_logit_pair
    dev = torch.device("cuda:0")
    cur, prev, _ = make_logit_pair(n=KL_ROWS, vocab=KL_VOCAB, dtype="bf16", seed=7)

    def to_dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)

    c0, p0 = to_dev(cur), to_dev(prev)
    pair_bytes = 2 * c0.numel() * 2
    n_copies = max(1, int(math.ceil(args.cold_bytes * (1 << 30) / pair_bytes)))
    cs = [c0] + [c0.clone() for _ in range(n_copies - 1)]
    ps = [p0] + [p0.clone() for _ in range(n_copies - 1)]
    kl = torch.empty(KL_ROWS, device=dev)
    locked = torch.zeros(KL_ROWS, device=dev, dtype=torch.uint8)
    eps = 1e-3
    if args.probe:
        for i in range(2 * n_copies):
            ba.ba_kl_lock(cs[i % n_copies], ps[i % n_copies], eps=eps, kl=kl, locked=locked)
        torch.cuda.synchronize()
        src = torch.ones(COPY_PROBE_BYTES // 4, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"probe": args.workload, "kl_passes": 2 * n_copies,
                          "copy_bytes_each": COPY_PROBE_BYTES, "copies": 4}), flush=True)
        return
    stream = torch.cuda.current_stream()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(n_copies):
                ba.ba_kl_lock(cs[i], ps[i], eps=eps, kl=kl, locked=locked, stream=torch.cuda.current_stream())
    stream.wait_stream(side)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    us = e0.elapsed_time(e1) * 1e3 / (args.steps * n_copies)
    nbytes = pair_bytes + KL_ROWS * (4 + 1 + 1)
    roof, achieved, _ = roofline_of(nbytes, 1, us)
    if not args.no_peaks:
        roof = with_measured(roof, measured_peaks(dev))
    out = {
        "metric": METRIC, "value": round(nbytes / (us * 1e-6) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": 1, "ms_per_step": round(us * 1e-3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic, seeded (workloads.make_logit_pair), resident in HBM",
        "config": {"workload": f"kl_lock: {KL_ROWS} token rows x {KL_VOCAB} vocabulary entries, two steps' bf16 "
                               f"logits, eps {eps}",
                   "bench_step": "one lock-criterion pass (KL per row and the lock update)",
                   "copies": n_copies},
        "latency_us": {"kl_pass": round(us, 2)},
        "roofline": {"kernel": "kl_lock_kernel", **roof,
                     "traffic": measured_traffic(None, "kl_lock", KL_SOURCES),
                     "algorithmic_bytes_per_launch": nbytes},
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        import oracle
        cores = host_cores()
        rows = 64
        t0 = time.perf_counter()
        oracle.kl_rows(oracle.to_f64(cur[:rows], "bf16"), oracle.to_f64(prev[:rows], "bf16"))
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": nbytes * rows / KL_ROWS / dt / 1e9, "unit": "GB/s",
                               "cores": cores["blas_threads"], **cores, "kind": "oracle",
                               "sample": f"{rows} of {KL_ROWS} rows, NumPy float64, {dt:.2f} s"}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50, help="timed block schedules")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c3_gqa_long")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured copy and GEMM peaks (kernel traces of the path alone)")
    ap.add_argument("--cold-bytes", type=float, default=1.0, help="GiB of rotated prefix copies")
    ap.add_argument("--lp", type=int, default=None,
                    help="prefix length override for the dense shapes (long-context sweep)")
    ap.add_argument("--gate", choices=["count", "count_cum", "cosine", "partial"], default=None,
                    help="gate override for the block schedule (count since the last refresh, per-head "
                         "cosine, or per-row partial refresh)")
    ap.add_argument("--sparse", type=float, default=None,
                    help="key-block density: time sparse-attention residual reuse instead of the block schedule")
    ap.add_argument("--probe", action="store_true",
                    help="counter-collection mode: only the prefix pass, eagerly, over the rotated copies, "
                         "then a plain device copy of known size (the counters' scale reference)")
    ap.add_argument("--update-mask", action="store_true",
                    help="count gates: feed the gate the generator's record of the rewritten positions (the "
                         "update mask a sampler holds) instead of comparing the block rows")
    ap.add_argument("--probe-inblock", action="store_true",
                    help="counter-collection mode for the in-block part alone: 4 eager ba_block_attn calls "
                         "with the cache merge (after one prefix pass fills the cache)")
    ap.add_argument("--yardstick", action="store_true",
                    help="time torch's fused attention (flash backend) on the prefix-pass shape beside the "
                         "library's prefix pass, instead of the block schedule (dense workloads)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; "
                                   f"--gpus {args.gpus} is not supported"}), flush=True)
        sys.exit(2)

    from workloads.synth import VARLEN_PRESETS
    if args.workload in VARLEN_PRESETS:
        run_varlen(args)
        return
    if args.workload == "kl_lock":
        run_kl(args)
        return

    import numpy as np
    import torch
    import cached_split_attention_amd as ba
    from workloads import preset

    dev = torch.device("cuda:0")

    def progress(msg):
        print(f"[bench {args.workload}] {msg}", file=sys.stderr, flush=True)

    over = {} if args.lp is None else dict(lp=args.lp)
    if args.gate is not None:
        over["gate"] = args.gate
    s = preset(args.workload, **over)
    progress(f"inputs drawn (prefix {s.lp})")

    def to_dev(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)

    kp0, vp0 = to_dev(s.kp), to_dev(s.vp)
    kv_bytes = 2 * kp0.numel() * 2
    n_copies = max(1, int(math.ceil(args.cold_bytes * (1 << 30) / kv_bytes)))
    kps = [kp0] + [kp0.clone() for _ in range(n_copies - 1)]
    vps = [vp0] + [vp0.clone() for _ in range(n_copies - 1)]
    q = [to_dev(x) for x in s.q]
    k = [to_dev(x) for x in s.k]
    v = [to_dev(x) for x in s.v]
    if args.probe:
        probe(args, s, q, kps, vps)
        return
    if args.yardstick:
        run_yardstick(args, s, q, kps, vps)
        return
    if args.probe_inblock:
        probe_inblock(args, s, q, k, v, kps, vps)
        return
    if args.sparse is not None:
        run_sparse(args, s, q, kps, vps)
        return
    attn = ba.CachedBlockAttention(kp0, vp0, nb=s.nb, hq=s.hq, gate=s.gate, tau=s.tau,
                                   gamma=s.gamma, scale=s.scale)
    stream = torch.cuda.current_stream()

    # untimed eager pass: record the (deterministic) decision pattern
    masks = None
    if args.update_mask:
        if s.gate not in ("count", "count_cum"):
            raise SystemExit("--update-mask needs a count gate")
        masks = [None] + [torch.from_numpy(s.rewritten[t]).to(dev) for t in range(1, s.steps + 1)]
    attn.start_block(kps[0], vps[0])
    decisions = [None]
    for t in range(1, s.steps + 1):
        attn.step(q[t], k[t], v[t], q[t - 1], k[t - 1], v[t - 1], upd_mask=None if masks is None else masks[t])
        decisions.append(attn.decision.cpu().numpy().copy())
        if attn.waits_given_up():
            raise RuntimeError(f"step {t}: a prefix workgroup gave up waiting for its gate")
    final_out = (attn.a_full.cpu().double().numpy().copy(), attn.l_full.cpu().double().numpy().copy())
    work = [step_work(s, decisions[t], mask=masks is not None) for t in range(1, s.steps + 1)]
    blk_bytes = sum(w[0] for w in work)
    blk_flops = sum(w[1] for w in work)
    rec_steps = [t for t in range(1, s.steps + 1) if (decisions[t] == 0).any()]
    reuse_steps = [t for t in range(2, s.steps + 1) if t not in rec_steps]

    progress(f"eager pass done, {len(rec_steps)} recompute steps")
    # one graph per prefix copy: the whole block schedule
    graphs = [attn.capture_block(q, k, v, kps[i], vps[i], masks=masks) for i in range(n_copies)]
    # single-step graphs for per-step latency
    g_rec = attn.capture(q, k, v, [1], new_block=True, kp=kps[0], vp=vps[0], masks=masks)
    # a reuse step repeated in place (same inputs, same decision, same
    # outputs) REUSE_REPS times in one graph, so the per-graph launch cost is
    # spread as it is over a block schedule
    g_reuse = (attn.capture(q, k, v, [reuse_steps[0]] * REUSE_REPS, new_block=False, masks=masks)
               if reuse_steps else None)

    def timed(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for i in range(args.warmup):
        graphs[(i + 1) % n_copies].replay()
    torch.cuda.synchronize()

    K = args.steps
    w0 = time.perf_counter()
    ms_per_step = timed(lambda i: graphs[(args.warmup + 1 + i) % n_copies].replay(), K)
    wall = time.perf_counter() - w0

    progress("block schedules timed")
    rec_us = timed(lambda i: g_rec.replay(), 20) * 1e3
    reuse_us = timed(lambda i: g_reuse.replay(), 10) * 1e3 / REUSE_REPS if g_reuse is not None else None

    # roofline leg: the prefix pass alone (every head recomputes), prefix
    # copies rotated so the K/V stream comes from HBM
    ws = torch.zeros(max(1, ba.ba_prefix_attn_workspace(q[1], kp0, vp0, scale=s.scale)), device=dev,
                     dtype=torch.uint8)
    a_tmp = torch.empty_like(attn.a_out)
    l_tmp = torch.empty_like(attn.l_out)
    # all copies' passes in one graph, so no per-replay launch latency is timed
    pgraph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(pgraph, stream=side):
            for i in range(n_copies):
                ba.ba_prefix_attn(q[1], kps[i], vps[i], a_tmp, l_tmp, ws, scale=s.scale,
                                  stream=torch.cuda.current_stream())
    stream.wait_stream(side)
    pgraph.replay()
    n_roof = 4
    pref_mean_us = timed(lambda i: pgraph.replay(), n_roof) * 1e3 / n_copies
    p_bytes1, p_flops1 = work[0][2], work[0][3]
    traffic = measured_traffic(args.workload)
    roof, achieved, achieved_tf = roofline_of(p_bytes1, p_flops1, pref_mean_us)
    if not args.no_peaks:
        roof = with_measured(roof, measured_peaks(dev))

    # in-block leg: the part every step computes (A_in/L_in over the block and
    # the fused merge with the cached prefix part into A_full/L_full), alone,
    # as ba_block_attn calls captured in one graph
    t_last = s.steps
    ib = {nm: torch.empty_like(attn.a_out) for nm in ("a_in", "a_full")}
    ib.update({nm: torch.empty_like(attn.l_out) for nm in ("l_in", "l_full")})
    n_ib = 16
    igraph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(igraph, stream=side):
            for _ in range(n_ib):
                ba.ba_block_attn(q[t_last], k[t_last], v[t_last], a_cache=attn.a_out, l_cache=attn.l_out,
                                 a_in=ib["a_in"], l_in=ib["l_in"], a_full=ib["a_full"], l_full=ib["l_full"],
                                 scale=s.scale, stream=torch.cuda.current_stream())
    stream.wait_stream(side)
    igraph.replay()
    ib_us = timed(lambda i: igraph.replay(), 4) * 1e3 / n_ib
    ib_flops = 4 * s.d * s.nb * s.nb * s.B * s.hq
    ib_bytes = (s.B * s.nb * s.hq * s.d * 2 + 2 * s.B * s.nb * s.hkv * s.d * 2
                + 2 * s.B * s.nb * s.hq * (s.d + 1) * 4 + s.B * s.nb * s.hq * (s.d + 1) * 4)
    inblock = {"kernel": "in-block attention with the fused merge (ba_block_attn, A_in/L_in and "
                         "A_full/L_full written)",
               "us": round(ib_us, 2), "algorithmic_flops": ib_flops, "algorithmic_bytes": ib_bytes,
               "tflops": round(ib_flops / (ib_us * 1e-6) / 1e12, 2),
               # (against the roof its arithmetic intensity reaches first: HBM for a
               # short block, the matrix cores for a long one)
               "roofline": roofline_of(ib_bytes, ib_flops, ib_us)[0],
               "gbs": round(ib_bytes / (ib_us * 1e-6) / 1e9, 1),
               "timing": f"{n_ib} calls in one graph, 4 replays, HIP events on the launching stream"}

    out = {
        "metric": METRIC,
        "value": round(blk_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic, seeded (workloads.preset), resident in HBM",
        "config": {"workload": f"{args.workload}: B={s.B} Hq={s.hq} Hkv={s.hkv} d={s.d} "
                               f"prefix={s.lp} block={s.nb} steps/block={s.steps} gate={s.gate}"
                               f" tau={s.tau} gamma={s.gamma}"
                               + (" gate_input=update_mask" if masks is not None else ""),
                   "bench_step": "one block schedule (every denoising step), replayed as a HIP graph",
                   "prefix_kv_copies": n_copies},
        "tflops": round(blk_flops / (ms_per_step * 1e-3) / 1e12, 4),
        "latency_us": {
            "mean_denoise_step": round(ms_per_step * 1e3 / s.steps, 2),
            "recompute_step": round(rec_us, 2),
            "reuse_step": round(reuse_us, 2) if reuse_us is not None else None,
            "prefix_pass": round(pref_mean_us, 2),
        },
        "recompute_steps_per_block": len(rec_steps),
        "roofline": {
            "kernel": "prefix pass (no valid cache: every head recomputes): split-KV attention kernel "
                      "+ split combine kernel, back to back",
            **roof,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": p_bytes1,
            "algorithmic_flops_per_launch": p_flops1,
            "gbs": round(achieved, 1),
            "tflops": round(achieved_tf, 3),
        },
        "inblock": inblock,
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        progress("CPU baseline (oracle on a bounded sample)")
        out["cpu_baseline"] = cpu_baseline(s, got=final_out if s.gate != "partial" else None)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
