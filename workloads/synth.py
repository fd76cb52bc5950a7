"""Seeded generators for the five workload shapes of block-diffusion attention.

Everything here is input preparation: i.i.d. normal draws, rounding to
bfloat16 (round to nearest even), step schedules that say which block rows a
denoising step rewrites, lock masks and branch lengths.  None of the method's
arithmetic (attention, log-space merge, reuse gate, varlen packing) lives here.

Layouts (element strides in brackets, head_dim contiguous):
  prefix K/V, dense   : [B, Hkv, Lp, d]
  block Q             : [B, Nb, Hq, d]
  block K/V           : [B, Nb, Hkv, d]
  varlen prefix K/V   : [H, sum(L_b), d]        (branch b owns rows cu_k[b]..)
  varlen block Q/K/V  : [sum(B_b), H, d]        (branch-major)
bfloat16 tensors are held as uint16 bit patterns; float32 ones as float32.

Draw order for a block schedule: Kp, Vp, block Q, K, V, then for each step in
order its update draws.  Varlen batch: prefix lengths, Kp, Vp, Q, K, V, lock
mask.
"""

from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np


# ----------------------------------------------------------------------------
# bfloat16 bit plumbing
# ----------------------------------------------------------------------------

def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bfloat16 bit patterns, round to nearest even.

    Inputs are finite (normal draws), so no NaN special case is needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    # Work in chunks so that multi-GiB tensors do not need a uint32 copy.
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_u.size, step):
        c = flat_u[s:s + step]
        lsb = (c >> np.uint32(16)) & np.uint32(1)
        flat_o[s:s + step] = ((c + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> exactly equal float32 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw(rng: np.random.Generator, shape, dtype: str, std: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if dtype == "bf16":
        return round_to_bf16_bits(x)
    return x


# ----------------------------------------------------------------------------
# dense block schedules (configs with one prefix per sequence)
# ----------------------------------------------------------------------------

@dataclass
class BlockSchedule:
    """Inputs of one block's denoising schedule.

    q[t], k[t], v[t] hold the block rows seen by step t (t = 1..steps);
    index 0 is the block as drawn before step 1.  touched[t, b] is how many
    block positions of sequence b the generator rewrote going from t-1 to t
    (the generator's own record, kept apart from any comparison of rows);
    rewritten[t, b, p] is 1 where position p was one of them (the update mask
    a sampler knows without comparing rows).
    """

    name: str
    dtype: str
    B: int
    hq: int
    hkv: int
    d: int
    lp: int
    nb: int
    steps: int
    scale: float
    gate: str          # "count", "count_cum" (since the last refresh) or "cosine"
    tau: int
    gamma: float
    seed: int
    kp: np.ndarray
    vp: np.ndarray
    q: list = field(default_factory=list)
    k: list = field(default_factory=list)
    v: list = field(default_factory=list)
    touched: np.ndarray = None
    rewritten: np.ndarray = None
    sigma: np.ndarray = None     # cosine schedules: per (step, head) noise level

    @property
    def group(self) -> int:
        return self.hq // self.hkv


def make_block_schedule(*, name="custom", dtype="bf16", B=1, hq=4, hkv=4, d=128,
                        lp=256, nb=32, steps=4, std=1.0, schedule="redraw",
                        redraw_range=(1, 4), unmask_range=(1, 2), poisson_lam=3.0,
                        sigma_range=(0.01, 0.5), gate="count", tau=4, gamma=0.95,
                        scale=None, seed=0) -> BlockSchedule:
    """Draw a prefix, an initial block and `steps` block updates.

    schedule:
      "redraw"  each step rewrites r ~ U{redraw_range} distinct positions
                drawn from all Nb (Q, K and V rows of every head);
      "unmask"  each step unmasks r ~ U{unmask_range} positions from the ones
                still masked (min(r, remaining)), rewriting their rows;
      "poisson" each step rewrites M ~ Poisson(lam) distinct positions per
                sequence, clamped to Nb;
      "qnoise"  each step adds sigma[t, h] * N(0, 1) to every block Q value
                in float32 and rounds back (K and V never change); sigma is
                drawn U(sigma_range) per (step, head).
      "none"    the block never changes.
    """
    if hq % hkv:
        raise ValueError("hq must be a multiple of hkv")
    rng = np.random.default_rng(seed)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    kp = _draw(rng, (B, hkv, lp, d), dtype, std)
    vp = _draw(rng, (B, hkv, lp, d), dtype, std)
    q0 = _draw(rng, (B, nb, hq, d), dtype, std)
    k0 = _draw(rng, (B, nb, hkv, d), dtype, std)
    v0 = _draw(rng, (B, nb, hkv, d), dtype, std)
    sch = BlockSchedule(name=name, dtype=dtype, B=B, hq=hq, hkv=hkv, d=d, lp=lp,
                        nb=nb, steps=steps, scale=float(scale), gate=gate, tau=int(tau),
                        gamma=float(gamma), seed=seed, kp=kp, vp=vp)
    sch.q.append(q0)
    sch.k.append(k0)
    sch.v.append(v0)
    touched = np.zeros((steps + 1, B), dtype=np.int32)
    rewritten = np.zeros((steps + 1, B, nb), dtype=np.uint8)
    masked = [list(range(nb)) for _ in range(B)]
    sigma = np.zeros((steps + 1, hq), dtype=np.float64) if schedule == "qnoise" else None

    for t in range(1, steps + 1):
        qp, kpv, vpv = sch.q[-1], sch.k[-1], sch.v[-1]
        if schedule == "qnoise":
            sig = rng.uniform(sigma_range[0], sigma_range[1], size=hq)
            sigma[t] = sig
            eps = rng.standard_normal(size=qp.shape, dtype=np.float32)
            base = bf16_bits_to_f32(qp) if dtype == "bf16" else qp
            newq = base + eps * sig.astype(np.float32)[None, None, :, None]
            newq = round_to_bf16_bits(newq) if dtype == "bf16" else newq.astype(np.float32)
            sch.q.append(newq)
            sch.k.append(kpv)
            sch.v.append(vpv)
            touched[t, :] = nb
            rewritten[t] = 1
            continue
        if schedule == "none":
            sch.q.append(qp)
            sch.k.append(kpv)
            sch.v.append(vpv)
            continue
        nq, nk, nv = qp.copy(), kpv.copy(), vpv.copy()
        for b in range(B):
            if schedule == "redraw":
                r = int(rng.integers(redraw_range[0], redraw_range[1] + 1))
                pos = rng.choice(nb, size=min(r, nb), replace=False)
            elif schedule == "unmask":
                r = int(rng.integers(unmask_range[0], unmask_range[1] + 1))
                r = min(r, len(masked[b]))
                if r > 0:
                    pick = rng.choice(len(masked[b]), size=r, replace=False)
                    pos = np.array(sorted(masked[b][i] for i in pick), dtype=np.int64)
                    chosen = set(pos.tolist())
                    masked[b] = [p for p in masked[b] if p not in chosen]
                else:
                    pos = np.zeros(0, dtype=np.int64)
            elif schedule == "poisson":
                r = min(int(rng.poisson(poisson_lam)), nb)
                pos = rng.choice(nb, size=r, replace=False)
            else:
                raise ValueError(f"unknown schedule {schedule!r}")
            pos = np.sort(np.asarray(pos, dtype=np.int64))
            touched[t, b] = pos.size
            rewritten[t, b, pos] = 1
            if pos.size:
                nq[b, pos] = _draw(rng, (pos.size, hq, d), dtype, std)
                nk[b, pos] = _draw(rng, (pos.size, hkv, d), dtype, std)
                nv[b, pos] = _draw(rng, (pos.size, hkv, d), dtype, std)
        sch.q.append(nq)
        sch.k.append(nk)
        sch.v.append(nv)
    sch.touched = touched
    sch.rewritten = rewritten
    sch.sigma = sigma
    return sch


# ----------------------------------------------------------------------------
# multi-branch varlen batch
# ----------------------------------------------------------------------------

@dataclass
class VarlenBatch:
    """Branches of one request, each with its own prefix and block.

    locked[p] = 1 marks a block position that no longer issues a query but is
    still attended as a key.  Branch b's block rows are rows
    sum(block_sizes[:b]) .. of q/k/v; its prefix rows are rows
    sum(prefix_lens[:b]) .. of kp/vp (per head).
    """

    name: str
    dtype: str
    h: int
    d: int
    scale: float
    seed: int
    block_sizes: np.ndarray
    prefix_lens: np.ndarray
    kp: np.ndarray      # [H, sum L, d]
    vp: np.ndarray
    q: np.ndarray       # [sum B, H, d]
    k: np.ndarray
    v: np.ndarray
    locked: np.ndarray  # uint8 [sum B]


def make_varlen_batch(*, name="custom", dtype="bf16", block_sizes=(4, 8, 16, 32, 64, 128),
                      prefix_range=(2048, 8192), prefix_lens=None, h=32, d=128, std=None,
                      lock_p=0.3, locked=None, scale=None, seed=0) -> VarlenBatch:
    rng = np.random.default_rng(seed)
    bs = np.asarray(block_sizes, dtype=np.int32)
    if prefix_lens is None:
        pl = rng.integers(prefix_range[0], prefix_range[1] + 1, size=bs.size).astype(np.int32)
    else:
        pl = np.asarray(prefix_lens, dtype=np.int32)
    if std is None:
        std = 1.0 / math.sqrt(d)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ltot, btot = int(pl.sum()), int(bs.sum())
    kp = _draw(rng, (h, ltot, d), dtype, std)
    vp = _draw(rng, (h, ltot, d), dtype, std)
    q = _draw(rng, (btot, h, d), dtype, std)
    k = _draw(rng, (btot, h, d), dtype, std)
    v = _draw(rng, (btot, h, d), dtype, std)
    if locked is None:
        lk = (rng.random(btot) < lock_p).astype(np.uint8)
    else:
        lk = np.asarray(locked, dtype=np.uint8)
    return VarlenBatch(name=name, dtype=dtype, h=h, d=d, scale=float(scale), seed=seed,
                       block_sizes=bs, prefix_lens=pl, kp=kp, vp=vp, q=q, k=k, v=v, locked=lk)


# ----------------------------------------------------------------------------
# the five workload shapes
# ----------------------------------------------------------------------------

PRESETS = {
    # Single layer, fp32, d=64: 4 heads, prefix 256, block 32, 8 steps that each
    # redraw 1-4 block rows; count gate with tau = 4.
    "c1_tiny_f32": dict(dtype="f32", B=1, hq=4, hkv=4, d=64, lp=256, nb=32, steps=8,
                        std=1.0, schedule="redraw", redraw_range=(1, 4), gate="count",
                        tau=4, seed=1),
    # LLaDA-8B-like: 32 heads, d=128, prefix 4096, block 32, 32 steps unmasking
    # 1-2 tokens each; count gate with tau = 4.
    "c2_llada": dict(dtype="bf16", B=1, hq=32, hkv=32, d=128, lp=4096, nb=32, steps=32,
                     std=1.0 / math.sqrt(128), schedule="unmask", unmask_range=(1, 2),
                     gate="count", tau=4, seed=2),
    # Long-context GQA: batch 8, 32 query heads on 8 KV heads, prefix 32768,
    # block 64, 64 steps with Poisson(3) updates; count gate with tau = 8.
    "c3_gqa_long": dict(dtype="bf16", B=8, hq=32, hkv=8, d=128, lp=32768, nb=64, steps=64,
                        std=1.0 / math.sqrt(128), schedule="poisson", poisson_lam=3.0,
                        gate="count", tau=8, seed=3),
    # Video-like: 24 heads, block 1560, prefix 31200, 8 steps of per-head
    # Gaussian noise on Q; cosine gate with gamma = 0.95 per head.
    "c4_video": dict(dtype="bf16", B=1, hq=24, hkv=24, d=128, lp=31200, nb=1560, steps=8,
                     std=1.0, schedule="qnoise", sigma_range=(0.01, 0.5), gate="cosine",
                     gamma=0.95, seed=4),
}

VARLEN_PRESETS = {
    # Six branches (block sizes 4..128), prefixes U[2048, 8192], 32 heads,
    # d = 128, Bernoulli(0.3) lock mask.
    "c5_varlen": dict(dtype="bf16", block_sizes=(4, 8, 16, 32, 64, 128),
                      prefix_range=(2048, 8192), h=32, d=128, lock_p=0.3, seed=5),
}


def make_key_block_lists(*, B: int, hkv: int, lp: int, density: float, block_keys: int = 64, seed: int = 0):
    """Selected and complementary key-block lists for a sparse attention over
    a prefix of lp keys: per (sequence, KV head), round(density * n) of the
    n = ceil(lp / block_keys) blocks, chosen uniformly at random (a seeded
    stand-in for a sparse-attention method's top-k selection), ascending.
    Returns int32 arrays [B, hkv, k] and [B, hkv, n - k]."""
    rng = np.random.default_rng(seed)
    n = (lp + block_keys - 1) // block_keys
    k = int(round(density * n))
    sel = np.empty((B, hkv, k), dtype=np.int32)
    rest = np.empty((B, hkv, n - k), dtype=np.int32)
    for b in range(B):
        for g in range(hkv):
            perm = rng.permutation(n)
            sel[b, g] = np.sort(perm[:k])
            rest[b, g] = np.sort(perm[k:])
    return sel, rest


def make_logit_pair(*, n: int, vocab: int, dtype: str = "bf16", std: float = 3.0,
                    drift_range=(1e-3, 1.0), seed: int = 0):
    """Two steps' logits for n token rows over a vocabulary: cur ~ N(0, std^2)
    i.i.d.; prev = cur + sigma_r * N(0, 1), with a per-row drift sigma_r drawn
    log-uniformly from drift_range (so the rows span converged and moving
    tokens).  Returns (cur, prev, sigma) as [n, vocab] arrays (bf16 bit
    patterns or float32) and the float64 sigmas."""
    rng = np.random.default_rng(seed)
    cur = rng.standard_normal((n, vocab), dtype=np.float32) * np.float32(std)
    lo, hi = math.log(drift_range[0]), math.log(drift_range[1])
    sigma = np.exp(rng.uniform(lo, hi, size=n))
    prev = cur + (rng.standard_normal((n, vocab), dtype=np.float32) * sigma[:, None].astype(np.float32))
    if dtype == "bf16":
        return round_to_bf16_bits(cur), round_to_bf16_bits(prev), sigma
    return cur, prev.astype(np.float32), sigma


def preset(name: str, **overrides):
    """Build one of the named workloads; keyword overrides replace fields."""
    if name in PRESETS:
        kw = dict(PRESETS[name])
        kw.update(overrides)
        return make_block_schedule(name=name, **kw)
    if name in VARLEN_PRESETS:
        kw = dict(VARLEN_PRESETS[name])
        kw.update(overrides)
        return make_varlen_batch(name=name, **kw)
    raise KeyError(name)
