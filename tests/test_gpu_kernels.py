"""GPU parity of each C-ABI entry point against the CPU oracle, on seeded
inputs small enough for the oracle yet spanning several tiles with ragged
tails, plus the edge cases (empty prefix, empty branches, all locked, ties,
NaN-poisoned cache, guard bands, determinism)."""

import math

import numpy as np
import pytest
import torch

import oracle
from workloads import (make_block_schedule, make_key_block_lists, make_logit_pair, make_varlen_batch,
                       round_to_bf16_bits)
from tests.gpu_util import DEV, check_a, check_l, dev_bits, dev_f32, dev_in, host

pytestmark = pytest.mark.gpu

ba = pytest.importorskip("cached_split_attention_amd")


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def f64(x, dtype):
    return oracle.to_f64(x, dtype)


# ----------------------------------------------------------------------------
# ba_lse_merge
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("d", [64, 96, 128, 132, 512, 1024])
def test_lse_merge(d):
    r = np.random.default_rng(40 + d)
    rows = 1237
    a1 = r.standard_normal((rows, d)).astype(np.float32)
    a2 = r.standard_normal((rows, d)).astype(np.float32)
    l1 = (r.standard_normal(rows) * 5).astype(np.float32)
    l2 = (r.standard_normal(rows) * 5).astype(np.float32)
    l1[::7] = -np.inf
    l2[::11] = -np.inf
    a1[::7] = 0.0
    a2[::11] = 0.0
    l1[3], l2[3] = 700.0, -700.0  # extreme gap
    wa, wl = oracle.merge(a1, l1, a2, l2)
    ga = torch.empty(rows, d, device=DEV)
    gl = torch.empty(rows, device=DEV)
    ba.ba_lse_merge(dev_f32(a1), dev_f32(l1), dev_f32(a2), dev_f32(l2), ga, gl)
    torch.cuda.synchronize()
    np.testing.assert_allclose(host(ga), wa, atol=2e-6, rtol=0)
    got_l = host(gl)
    assert np.array_equal(np.isneginf(got_l), np.isneginf(wl))
    fin = ~np.isneginf(wl)
    np.testing.assert_allclose(got_l[fin], wl[fin], atol=2e-5 * max(1, np.abs(wl[fin]).max() / 100), rtol=0)
    # in place into the first operand, and into the second: A and L (a
    # row's threads span two waves whenever d/4 does not divide 64)
    for into in (1, 2):
        x1, y1, x2, y2 = dev_f32(a1), dev_f32(l1), dev_f32(a2), dev_f32(l2)
        xa, xl = (x1, y1) if into == 1 else (x2, y2)
        ba.ba_lse_merge(x1, y1, x2, y2, xa, xl)
        torch.cuda.synchronize()
        np.testing.assert_allclose(host(xa), wa, atol=2e-6, rtol=0, err_msg=f"in place into operand {into}")
        got_l = host(xl)
        assert np.array_equal(np.isneginf(got_l), np.isneginf(wl)), f"in place into operand {into}"
        np.testing.assert_allclose(got_l[fin], wl[fin], atol=2e-5 * max(1, np.abs(wl[fin]).max() / 100), rtol=0,
                                   err_msg=f"in place L into operand {into}")


# ----------------------------------------------------------------------------
# ba_reuse_gate
# ----------------------------------------------------------------------------

def _gate_count_run(s, slicer=None, use_mask=False):
    q = [dev_in(x, s.dtype) for x in s.q]
    k = [dev_in(x, s.dtype) for x in s.k]
    v = [dev_in(x, s.dtype) for x in s.v]
    if slicer is not None:
        q, k, v = [slicer(x) for x in q], [slicer(x) for x in k], [slicer(x) for x in v]
    ref = oracle.step_gates(s)
    ws = torch.zeros(ba.ba_reuse_gate_workspace(ba.BA_GATE_COUNT, q[1], q[0], k_cur=k[1], k_prev=k[0],
                                                v_cur=v[1], v_prev=v[0]), device=DEV, dtype=torch.uint8)
    dec = torch.empty(s.B, s.hq, device=DEV, dtype=torch.uint8)
    m = torch.empty(s.B, device=DEV, dtype=torch.int32)
    for t in range(1, s.steps + 1):
        if use_mask:
            mask = torch.from_numpy(oracle.updated_positions([s.q[t], s.k[t], s.v[t]],
                                                             [s.q[t - 1], s.k[t - 1], s.v[t - 1]])
                                    .astype(np.uint8)).to(DEV)
            ba.ba_reuse_gate(ba.BA_GATE_COUNT, q[t], q[t - 1], upd_mask=mask, tau=s.tau,
                             cache_valid=t > 1, m_count=m, decision=dec, workspace=ws)
        else:
            ba.ba_reuse_gate(ba.BA_GATE_COUNT, q[t], q[t - 1], k_cur=k[t], k_prev=k[t - 1], v_cur=v[t],
                             v_prev=v[t - 1], tau=s.tau, cache_valid=t > 1, m_count=m, decision=dec,
                             workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(m.cpu().numpy(), ref[t]["m"]), (t, m.cpu().numpy(), ref[t]["m"])
        assert np.array_equal(m.cpu().numpy(), s.touched[t])
        assert np.array_equal(dec.cpu().numpy(), ref[t]["decision"]), t
        assert not ws.any(), "gate workspace must be zero again after the call"


@pytest.mark.parametrize("dtype,schedule", [("bf16", "redraw"), ("bf16", "poisson"), ("f32", "unmask"),
                                            ("bf16", "unmask")])
def test_gate_count(dtype, schedule):
    s = make_block_schedule(dtype=dtype, B=3, hq=6, hkv=2, d=64, lp=8, nb=24, steps=10,
                            schedule=schedule, redraw_range=(0, 5), poisson_lam=3.0,
                            unmask_range=(1, 3), gate="count", tau=3, seed=50)
    _gate_count_run(s)


def test_gate_count_unaligned_rows_and_mask():
    # head dim 66 sliced to 64 from position 1: rows start 2 bytes off 16
    s = make_block_schedule(dtype="bf16", B=2, hq=2, hkv=2, d=66, lp=8, nb=16, steps=6,
                            schedule="redraw", redraw_range=(0, 3), gate="count", tau=2, seed=51)
    # compare only elements 1..64: changes are whole-row redraws, so counts agree
    _gate_count_run(s, slicer=lambda x: x[..., 1:65])
    _gate_count_run(s, use_mask=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gate_cosine(dtype):
    s = make_block_schedule(dtype=dtype, B=2, hq=5, hkv=5, d=64, lp=8, nb=37, steps=5, std=1.0,
                            schedule="qnoise", sigma_range=(0.01, 0.6), gate="cosine", gamma=0.95,
                            seed=52)
    ref = oracle.step_gates(s)
    q = [dev_in(x, dtype) for x in s.q]
    ws = torch.zeros(ba.ba_reuse_gate_workspace(ba.BA_GATE_COSINE, q[1], q[0]), device=DEV, dtype=torch.uint8)
    dec = torch.empty(s.B, s.hq, device=DEV, dtype=torch.uint8)
    cos = torch.empty(s.B, s.hq, device=DEV, dtype=torch.float64)
    saw = set()
    for t in range(1, s.steps + 1):
        ba.ba_reuse_gate(ba.BA_GATE_COSINE, q[t], q[t - 1], gamma=s.gamma, cache_valid=t > 1, cos=cos,
                         decision=dec, workspace=ws)
        torch.cuda.synchronize()
        c = cos.cpu().numpy()
        assert np.abs(c - ref[t]["cos"]).max() <= 1e-13, np.abs(c - ref[t]["cos"]).max()
        assert np.array_equal(dec.cpu().numpy(), ref[t]["decision"]), t
        saw |= set(dec.cpu().numpy().ravel().tolist()) if t > 1 else set()
        assert not ws.any()
    assert saw == {0, 1}, "schedule should exercise both decisions"


def test_gate_cosine_exact_tie_and_zero_norm():
    d = 64
    q = np.zeros((1, 1, 3, d), dtype=np.float32)
    p = np.zeros((1, 1, 3, d), dtype=np.float32)
    q[0, 0, 0, :2] = [3, 4]
    p[0, 0, 0, :2] = [4, 3]        # cos = 24/25 = 0.96 exactly
    q[0, 0, 1, :2] = [1, 2]
    p[0, 0, 1, :2] = [1, 2]        # cos = 1
    q[0, 0, 2, :] = 0.0            # zero norm
    p[0, 0, 2, :2] = [1, 1]
    for dtype in ("bf16", "f32"):
        qq = dev_bits(round_to_bf16_bits(q)) if dtype == "bf16" else dev_f32(q)
        pp = dev_bits(round_to_bf16_bits(p)) if dtype == "bf16" else dev_f32(p)
        ws = torch.zeros(ba.ba_reuse_gate_workspace(ba.BA_GATE_COSINE, qq, pp), device=DEV, dtype=torch.uint8)
        dec = torch.empty(1, 3, device=DEV, dtype=torch.uint8)
        cos = torch.empty(1, 3, device=DEV, dtype=torch.float64)
        for gamma, want in ((0.96, [0, 1, 0]), (0.9599, [1, 1, 0]), (-5.0, [1, 1, 0])):
            ba.ba_reuse_gate(ba.BA_GATE_COSINE, qq, pp, gamma=gamma, cache_valid=True, cos=cos, decision=dec,
                             workspace=ws)
            torch.cuda.synchronize()
            assert cos.cpu().numpy()[0, 0] == 0.96
            assert dec.cpu().numpy()[0].tolist() == want, (dtype, gamma)
        ba.ba_reuse_gate(ba.BA_GATE_COSINE, qq, pp, gamma=0.5, cache_valid=False, cos=cos, decision=dec,
                         workspace=ws)
        torch.cuda.synchronize()
        assert not dec.cpu().numpy().any()


def _random_split_shapes(n, seed):
    # (dtype, B, hq, hkv, d, lp, nb): batch 1-3, GQA group 1-4, head dim 64
    # or 128, prefixes from empty through ragged multi-split lengths, blocks
    # from one row to 300, so that every launch shape (few rows, 128-row and
    # 256-row tiles) and ragged tails come up.
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        hkv = int(r.choice([1, 2, 4]))
        g = int(r.integers(1, 5))
        lp = 0 if i % 5 == 4 else int(r.integers(1, 2600))
        nb = int(r.choice([1, int(r.integers(2, 40)), int(r.integers(40, 120)), int(r.integers(120, 301))]))
        dt = "f32" if i % 6 == 5 else "bf16"
        out.append((dt, int(r.integers(1, 4)), hkv * g, hkv, int(r.choice([64, 128])), lp, nb))
    return out


@pytest.mark.parametrize("case", _random_split_shapes(12, 2024))
def test_split_attn_random_shapes(case):
    # Seeded random shapes through the one-launch split attention, every head
    # recomputing: A_out, A_in and A_full against the oracle on all rows.
    dtype, B, hq, hkv, d, lp, nb = case
    print(f"case {case}", flush=True)
    s = _dense_inputs(dtype, B, hq, hkv, d, lp, nb, seed=B * 1000 + lp + nb)
    rows = B * nb
    if lp > 0:
        want_a, want_l = _oracle_prefix(s)
    else:
        want_a, want_l = np.zeros((rows, hq, d)), np.full((rows, hq), -np.inf)
    want_ai, want_li = _oracle_block(s)
    want_f, want_lf = oracle.merge(want_a, want_l, want_ai, want_li)
    q, k, v = dev_in(s.q[0], dtype), dev_in(s.k[0], dtype), dev_in(s.v[0], dtype)
    if lp > 0:
        kp, vp = dev_in(s.kp, dtype), dev_in(s.vp, dtype)
    else:
        kp = vp = torch.zeros(B, hkv, 0, d, device=DEV, dtype=q.dtype)
    ws = torch.zeros(max(1, ba.ba_prefix_attn_workspace(q, kp, vp)), device=DEV, dtype=torch.uint8)
    outs = [torch.full((rows, hq, d), 9.0, device=DEV) for _ in range(3)]
    ls = [torch.full((rows, hq), 9.0, device=DEV) for _ in range(3)]
    ba.ba_split_attn(q, kp, vp, k, v, outs[0], ls[0], outs[1], ls[1], outs[2], ls[2], ws)
    torch.cuda.synchronize()
    check_a(host(outs[0]), want_a, "A_out")
    check_l(host(ls[0]), want_l, "L_out")
    check_a(host(outs[1]), want_ai, "A_in")
    check_l(host(ls[1]), want_li, "L_in")
    check_a(host(outs[2]), want_f, "A_full")
    check_l(host(ls[2]), want_lf, "L_full")


# ----------------------------------------------------------------------------
# gate variants: count since the last refresh, per-row partial refresh
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("use_mask", [False, True])
def test_gate_count_cumulative(use_mask):
    # M since the last refresh, the decision and the kept marks at every step
    # of a schedule whose per-step counts stay below tau while the
    # cumulative ones cross it now and then.
    s = make_block_schedule(dtype="bf16", B=3, hq=4, hkv=2, d=64, lp=8, nb=16, steps=14,
                            schedule="redraw", redraw_range=(0, 2), gate="count_cum", tau=4, seed=53)
    q = [dev_in(x, s.dtype) for x in s.q]
    k = [dev_in(x, s.dtype) for x in s.k]
    v = [dev_in(x, s.dtype) for x in s.v]
    ref = oracle.step_gates(s)
    ws = torch.zeros(ba.ba_reuse_gate_workspace(ba.BA_GATE_COUNT_CUM, q[1], q[0], k_cur=k[1], k_prev=k[0],
                                                v_cur=v[1], v_prev=v[0]), device=DEV, dtype=torch.uint8)
    dec = torch.empty(s.B, s.hq, device=DEV, dtype=torch.uint8)
    m = torch.empty(s.B, device=DEV, dtype=torch.int32)
    since = torch.full((s.B, s.nb), 5, device=DEV, dtype=torch.uint8)   # stale: the first step clears it
    saw = set()
    for t in range(1, s.steps + 1):
        if use_mask:
            mask = torch.from_numpy(oracle.updated_positions([s.q[t], s.k[t], s.v[t]],
                                                             [s.q[t - 1], s.k[t - 1], s.v[t - 1]])
                                    .astype(np.uint8)).to(DEV)
            ba.ba_reuse_gate(ba.BA_GATE_COUNT_CUM, q[t], q[t - 1], upd_mask=mask, tau=s.tau, cache_valid=t > 1,
                             m_count=m, decision=dec, workspace=ws, since_refresh=since)
        else:
            ba.ba_reuse_gate(ba.BA_GATE_COUNT_CUM, q[t], q[t - 1], k_cur=k[t], k_prev=k[t - 1], v_cur=v[t],
                             v_prev=v[t - 1], tau=s.tau, cache_valid=t > 1, m_count=m, decision=dec,
                             workspace=ws, since_refresh=since)
        torch.cuda.synchronize()
        got_m, got_d = m.cpu().numpy(), dec.cpu().numpy()
        assert np.array_equal(got_m, ref[t]["m"]), (t, got_m, ref[t]["m"])
        assert np.array_equal(got_d, ref[t]["decision"]), t
        kept = since.cpu().numpy()
        assert set(np.unique(kept).tolist()) <= {0, 1}
        # marks: the count's positions while reusing, none after a recompute
        assert np.array_equal(kept.sum(axis=1), np.where(got_d[:, 0] == 1, got_m, 0)), t
        assert not ws.any()
        if t > 1:
            saw |= set(got_d[:, 0].tolist())
        assert (got_m >= s.touched[t]).all()
    assert saw == {0, 1}, "schedule should exercise both decisions"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gate_rows(dtype):
    # Rows mode: per position, is its Q row unchanged; K/V are not looked at.
    s = make_block_schedule(dtype=dtype, B=2, hq=3, hkv=3, d=64, lp=8, nb=40, steps=5, schedule="redraw",
                            redraw_range=(0, 6), seed=54)
    q = [dev_in(x, dtype) for x in s.q]
    ws = torch.zeros(ba.ba_reuse_gate_workspace(ba.BA_GATE_ROWS, q[1], q[0]), device=DEV, dtype=torch.uint8)
    keep = torch.empty(s.B, s.nb, device=DEV, dtype=torch.uint8)
    m = torch.empty(s.B, device=DEV, dtype=torch.int32)
    for t in range(1, s.steps + 1):
        ba.ba_reuse_gate(ba.BA_GATE_ROWS, q[t], q[t - 1], cache_valid=t > 1, m_count=m, decision=keep,
                         workspace=ws)
        torch.cuda.synchronize()
        ch = oracle.rows_changed(s.q[t], s.q[t - 1])
        assert np.array_equal(keep.cpu().numpy(), ((~ch) & (t > 1)).astype(np.uint8)), t
        assert np.array_equal(m.cpu().numpy(), ch.sum(axis=1)), t
        assert not ws.any()
    k = dev_in(s.k[1], dtype)
    with pytest.raises(ba.BaError):
        ba.ba_reuse_gate(ba.BA_GATE_ROWS, q[1], q[0], k_cur=k, k_prev=k, v_cur=k, v_prev=k, m_count=m,
                         decision=keep, workspace=ws)


ROWS_SHAPES = [
    # (B, hq, hkv, d, lp, nb): few rows per KV head with split-KV, GQA
    # 128-row tiles, the alternating kernel, head dim 64, one split
    (3, 8, 8, 128, 1500, 32),
    (2, 8, 2, 128, 2000, 64),
    (1, 4, 1, 128, 900, 80),
    (2, 6, 3, 64, 555, 41),
    (2, 4, 4, 128, 64, 24),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", ROWS_SHAPES)
def test_prefix_attn_rows(dtype, shape):
    # Listed rows recomputed into the cache; the others untouched.  Sequence
    # 0 lists a random subset, sequence 1 none (or all rows when it is the
    # last), the rest random; lists come from ba_varlen_pack.
    B, hq, hkv, d, lp, nb = shape
    if dtype == "f32" and lp > 1000:
        lp = 700
    s = _dense_inputs(dtype, B, hq, hkv, d, lp, nb, seed=lp + nb)
    want_a, want_l = _oracle_prefix(s)
    r = np.random.default_rng(nb)
    sel = r.random((B, nb)) < 0.3
    if B > 1:
        sel[1] = B == 2
    q, kp, vp = dev_in(s.q[0], dtype), dev_in(s.kp, dtype), dev_in(s.vp, dtype)
    keep = torch.from_numpy((~sel).astype(np.uint8).ravel()).to(DEV)
    cu = torch.empty(B + 1, device=DEV, dtype=torch.int32)
    rows = torch.empty(B * nb, device=DEV, dtype=torch.int32)
    total = torch.empty(1, device=DEV, dtype=torch.int32)
    ba.ba_varlen_pack([nb] * B, keep, cu, rows, total)
    ws = torch.zeros(max(1, ba.ba_prefix_attn_workspace(q, kp, vp)), device=DEV, dtype=torch.uint8)
    a = torch.full((B * nb, hq, d), 777.0, device=DEV)
    l = torch.full((B * nb, hq), 777.0, device=DEV)
    ba.ba_prefix_attn_rows(q, kp, vp, cu, rows, a, l, ws)
    torch.cuda.synchronize()
    assert int(total.item()) == int(sel.sum())
    flat = sel.ravel()
    ga, gl = host(a), host(l)
    check_a(ga[flat], want_a[flat], "A_out listed rows")
    check_l(gl[flat], want_l[flat], "L_out listed rows")
    assert (ga[~flat] == 777.0).all() and (gl[~flat] == 777.0).all(), "unlisted rows must stay untouched"
    # a hand-made list in another order, with a repeated row, gives the same
    # values for the rows it names
    order = [int(x) for x in np.flatnonzero(flat)[::-1]]
    if order:
        order.append(order[0])
        seq = np.array(order) // nb
        idx = np.argsort(seq, kind="stable")
        lst = np.array(order)[idx].astype(np.int32)
        cu2 = np.searchsorted(seq[idx], np.arange(B + 1)).astype(np.int32)
        a2 = torch.full_like(a, 777.0)
        l2 = torch.full_like(l, 777.0)
        ba.ba_prefix_attn_rows(q, kp, vp, torch.from_numpy(cu2).to(DEV), torch.from_numpy(lst).to(DEV), a2, l2, ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(a2)[flat], ga[flat])
        np.testing.assert_array_equal(host(l2)[flat], gl[flat])


# ----------------------------------------------------------------------------
# ba_varlen_pack
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("sizes,p_lock", [((4, 8, 16, 32, 64, 128), 0.3), ((3, 0, 5, 1, 0), 0.5),
                                          ((7, 9), 1.0), ((7, 9), 0.0), ((300, 1, 70), 0.3), ((), 0.3)])
def test_varlen_pack(sizes, p_lock):
    r = np.random.default_rng(len(sizes) + int(10 * p_lock))
    n = int(sum(sizes))
    locked = (r.random(n) < p_lock).astype(np.uint8)
    cu_w, gather_w, total_w = oracle.varlen_pack(locked, sizes)
    h, d = 3, 128
    q = r.standard_normal((max(n, 1), h, d)).astype(np.float32)
    qd = dev_bits(round_to_bf16_bits(q))
    cu = torch.full((len(sizes) + 1,), -7, device=DEV, dtype=torch.int32)
    gather = torch.full((max(n, 1),), -7, device=DEV, dtype=torch.int32)
    total = torch.full((1,), -7, device=DEV, dtype=torch.int32)
    packed = torch.zeros(max(n, 1), h, d, device=DEV, dtype=torch.bfloat16)
    ba.ba_varlen_pack(sizes, torch.from_numpy(locked).to(DEV) if n else torch.zeros(1, dtype=torch.uint8, device=DEV),
                      cu, gather, total, qd if n else None, packed if n else None)
    torch.cuda.synchronize()
    assert cu.cpu().numpy().tolist() == cu_w.tolist()
    assert int(total.item()) == total_w
    g = gather.cpu().numpy()
    assert g[:total_w].tolist() == gather_w.tolist()
    if n:
        assert np.all(g[total_w:n] == -1)
        got = packed.view(torch.int16).cpu().numpy()[:total_w]
        want = qd.view(torch.int16).cpu().numpy()[gather_w]
        assert np.array_equal(got, want)


# ----------------------------------------------------------------------------
# ba_prefix_attn / ba_block_attn, dense
# ----------------------------------------------------------------------------

def _dense_inputs(dtype, B, hq, hkv, d, lp, nb, seed, std=1.0):
    s = make_block_schedule(dtype=dtype, B=B, hq=hq, hkv=hkv, d=d, lp=lp, nb=nb, steps=0, std=std,
                            schedule="none", seed=seed)
    return s


def _oracle_prefix(s, t=0):
    out_a = np.zeros((s.B, s.nb, s.hq, s.d))
    out_l = np.zeros((s.B, s.nb, s.hq))
    for b in range(s.B):
        for h in range(s.hq):
            out_a[b, :, h], out_l[b, :, h] = oracle.prefix_rows(s, t, b, h)
    return out_a.reshape(s.B * s.nb, s.hq, s.d), out_l.reshape(s.B * s.nb, s.hq)


def _oracle_block(s, t=0):
    out_a = np.zeros((s.B, s.nb, s.hq, s.d))
    out_l = np.zeros((s.B, s.nb, s.hq))
    for b in range(s.B):
        for h in range(s.hq):
            out_a[b, :, h], out_l[b, :, h] = oracle.block_rows(s, t, b, h)
    return out_a.reshape(s.B * s.nb, s.hq, s.d), out_l.reshape(s.B * s.nb, s.hq)


DENSE_SHAPES = [
    # (B, hq, hkv, d, lp, nb): 128-row tiles with a ragged second tile, split-KV
    (1, 8, 2, 128, 777, 50),
    # 64-row tiles, GQA, split-KV with a ragged last chunk
    (2, 4, 2, 128, 1000, 20),
    # 32-row tiles (few rows per KV head)
    (3, 2, 2, 128, 300, 20),
    (1, 4, 4, 128, 64, 32),     # exactly one tile, one split
    (2, 6, 3, 64, 555, 41),     # head dim 64
    (1, 3, 1, 64, 129, 9),      # G = 3, 27 rows
    # 256-row alternating kernel: 200 rows (wave 7 idle, wave 6 ragged),
    # one 64-key tile per split with a ragged last split
    (1, 8, 2, 128, 1000, 50),
    # 520 rows: the last row tile has 8 rows (group 1 idle), 6 tiles
    (2, 4, 1, 128, 333, 130),
    # head dim 64, 300 rows
    (1, 2, 2, 64, 700, 300),
    # few splits of many tiles each: the 4-stage ring wraps several times
    (4, 16, 16, 128, 3000, 200),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", DENSE_SHAPES)
def test_prefix_attn(dtype, shape):
    B, hq, hkv, d, lp, nb = shape
    s = _dense_inputs(dtype, B, hq, hkv, d, lp, nb, seed=hash(shape) % 1000)
    want_a, want_l = _oracle_prefix(s)
    q, kp, vp = dev_in(s.q[0], dtype), dev_in(s.kp, dtype), dev_in(s.vp, dtype)
    ws = torch.zeros(max(1, ba.ba_prefix_attn_workspace(q, kp, vp)), device=DEV, dtype=torch.uint8)
    a = torch.full((B * nb, hq, d), 777.0, device=DEV)
    l = torch.full((B * nb, hq), 777.0, device=DEV)
    ba.ba_prefix_attn(q, kp, vp, a, l, ws)
    torch.cuda.synchronize()
    check_a(host(a), want_a, "A_out")
    check_l(host(l), want_l, "L_out")
    # bitwise deterministic
    a2 = torch.zeros_like(a)
    l2 = torch.zeros_like(l)
    ba.ba_prefix_attn(q, kp, vp, a2, l2, ws)
    torch.cuda.synchronize()
    assert torch.equal(a, a2) and torch.equal(l, l2)


@pytest.mark.parametrize("offset", [-10.0, -5.0])
@pytest.mark.parametrize("shape", [DENSE_SHAPES[0], DENSE_SHAPES[1], DENSE_SHAPES[2], DENSE_SHAPES[6],
                                   DENSE_SHAPES[9]])
def test_prefix_attn_score_jumps(offset, shape):
    """Scores that jump far above the running reference mid-row.  Prefix keys
    come in 96-key stripes; every other stripe (the first included) is
    shifted by `offset` along the queries' mean direction, so scores jump by
    about 80 (offset -10) or 40 (offset -5) log2 units between stripes.  A
    split whose first tile is in a low stripe then meets scores whose
    exponentials under the reference overflow a tile sum of 2^64 (the tile
    is redone under its maximum) or reach about 2^40 (kept as they are)."""
    from workloads import bf16_bits_to_f32
    B, hq, hkv, d, lp, nb = shape
    s = _dense_inputs("bf16", B, hq, hkv, d, lp, nb, seed=31 + int(-offset))
    kp = bf16_bits_to_f32(s.kp) * np.float32(0.3)
    kp[:, :, (np.arange(lp) // 96) % 2 == 0, :] += np.float32(offset)
    s.kp = round_to_bf16_bits(kp)
    s.q[0] = round_to_bf16_bits(bf16_bits_to_f32(s.q[0]) * np.float32(0.3) + np.float32(0.5))
    want_a, want_l = _oracle_prefix(s)
    q, kp_d, vp_d = dev_bits(s.q[0]), dev_bits(s.kp), dev_bits(s.vp)
    ws = torch.zeros(max(1, ba.ba_prefix_attn_workspace(q, kp_d, vp_d)), device=DEV, dtype=torch.uint8)
    a = torch.full((B * nb, hq, d), 777.0, device=DEV)
    l = torch.full((B * nb, hq), 777.0, device=DEV)
    ba.ba_prefix_attn(q, kp_d, vp_d, a, l, ws)
    torch.cuda.synchronize()
    check_a(host(a), want_a, "A_out")
    check_l(host(l), want_l, "L_out")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(3, 6, 2, 128, 900, 33), (3, 8, 2, 128, 700, 70)])
def test_prefix_attn_decision_leaves_cache_untouched(dtype, shape):
    # the second shape (280 rows per KV head) runs the 256-row kernel
    B, hq, hkv, d, lp, nb = shape
    s = _dense_inputs(dtype, B, hq, hkv, d, lp, nb, seed=61)
    want_a, want_l = _oracle_prefix(s)
    r = np.random.default_rng(3)
    dec = (r.random((B, hq)) < 0.5).astype(np.uint8)
    dec[0, :] = 1            # a whole sequence reused
    dec[1, :] = 0            # a whole sequence recomputed
    q, kp, vp = dev_in(s.q[0], dtype), dev_in(s.kp, dtype), dev_in(s.vp, dtype)
    ws = torch.zeros(max(1, ba.ba_prefix_attn_workspace(q, kp, vp)), device=DEV, dtype=torch.uint8)
    a = torch.full((B * nb, hq, d), 123.0, device=DEV)
    l = torch.full((B * nb, hq), -55.0, device=DEV)
    ba.ba_prefix_attn(q, kp, vp, a, l, ws, decision=torch.from_numpy(dec).to(DEV))
    torch.cuda.synchronize()
    ga, gl = host(a).reshape(B, nb, hq, d), host(l).reshape(B, nb, hq)
    wa, wl = want_a.reshape(B, nb, hq, d), want_l.reshape(B, nb, hq)
    for b in range(B):
        for h in range(hq):
            if dec[b, h]:
                assert np.all(ga[b, :, h] == 123.0) and np.all(gl[b, :, h] == -55.0)
            else:
                check_a(ga[b, :, h], wa[b, :, h], f"A_out b{b} h{h}")
                check_l(gl[b, :, h], wl[b, :, h], f"L_out b{b} h{h}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(3, 6, 2, 128, 900, 33), (1, 4, 4, 128, 64, 32), (3, 8, 2, 128, 700, 70),
                                   (2, 6, 3, 64, 555, 41), (2, 4, 2, 128, 0, 20)])
def test_prefix_attn_merge(dtype, shape):
    # Prefix pass fused with the merge against a precomputed in-block part:
    # recomputed heads merge fresh A_out/L_out, reused heads the cached ones
    # (left untouched); split and single-pass plans, the 256-row kernel, d=64
    # and an empty prefix.
    B, hq, hkv, d, lp, nb = shape
    s = _dense_inputs(dtype, B, hq, hkv, d, lp, nb, seed=71)
    rows = B * nb
    if lp > 0:
        want_a, want_l = _oracle_prefix(s)
    else:
        want_a, want_l = np.zeros((rows, hq, d)), np.full((rows, hq), -np.inf)
    r = np.random.default_rng(9)
    a_in = r.standard_normal((rows, hq, d)).astype(np.float32)
    l_in = (r.standard_normal((rows, hq)) * 3 + 2).astype(np.float32)
    l_in[::7, 0] = -np.inf
    a_in[::7, 0] = 0.0
    cache_a = r.standard_normal((rows, hq, d)).astype(np.float32)
    cache_l = r.standard_normal((rows, hq)).astype(np.float32)
    dec = (r.random((B, hq)) < 0.5).astype(np.uint8)
    dec[0, 0] = 0
    exp_a, exp_l = want_a.copy(), want_l.copy()
    for b in range(B):
        for h in range(hq):
            if dec[b, h]:
                exp_a[b * nb:(b + 1) * nb, h] = cache_a[b * nb:(b + 1) * nb, h]
                exp_l[b * nb:(b + 1) * nb, h] = cache_l[b * nb:(b + 1) * nb, h]
    want_f, want_lf = oracle.merge(exp_a, exp_l, a_in, l_in)
    q = dev_in(s.q[0], dtype)
    if lp > 0:
        kp, vp = dev_in(s.kp, dtype), dev_in(s.vp, dtype)
    else:
        kp = vp = torch.zeros(B, hkv, 0, d, device=DEV, dtype=q.dtype)
    ws = torch.zeros(max(1, ba.ba_prefix_attn_workspace(q, kp, vp)), device=DEV, dtype=torch.uint8)
    a_out = torch.from_numpy(cache_a).to(DEV)
    l_out = torch.from_numpy(cache_l).to(DEV)
    a_full = torch.full((rows, hq, d), 5.0, device=DEV)
    l_full = torch.full((rows, hq), 5.0, device=DEV)
    ba.ba_prefix_attn_merge(q, kp, vp, a_out, l_out, torch.from_numpy(a_in).to(DEV),
                            torch.from_numpy(l_in).to(DEV), a_full, l_full, ws,
                            decision=torch.from_numpy(dec).to(DEV))
    torch.cuda.synchronize()
    ga, gl = host(a_out), host(l_out)
    for b in range(B):
        for h in range(hq):
            sl = slice(b * nb, (b + 1) * nb)
            if dec[b, h]:
                assert np.array_equal(ga[sl, h], cache_a[sl, h]) and np.array_equal(gl[sl, h], cache_l[sl, h])
            else:
                check_a(ga[sl, h], want_a[sl, h], f"A_out b{b} h{h}")
                check_l(gl[sl, h], want_l[sl, h], f"L_out b{b} h{h}")
    check_a(host(a_full), want_f, "A_full")
    check_l(host(l_full), want_lf, "L_full")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(3, 6, 2, 128, 900, 33), (1, 4, 4, 128, 64, 32), (3, 8, 2, 128, 700, 70),
                                   (2, 6, 3, 64, 555, 41), (2, 4, 2, 128, 0, 20), (1, 2, 2, 128, 400, 100)])
def test_split_attn(dtype, shape):
    # Prefix and in-block parts in one launch, then combine and merge: the
    # in-block result, fresh A_out of recomputed heads (cached ones left
    # alone) and A_full against the oracle; both parts' shapes (few rows, 128
    # and 256-row tiles, d=64, empty prefix) and a gate decision.
    B, hq, hkv, d, lp, nb = shape
    s = _dense_inputs(dtype, B, hq, hkv, d, lp, nb, seed=81)
    rows = B * nb
    if lp > 0:
        want_a, want_l = _oracle_prefix(s)
    else:
        want_a, want_l = np.zeros((rows, hq, d)), np.full((rows, hq), -np.inf)
    want_ai, want_li = _oracle_block(s)
    r = np.random.default_rng(12)
    cache_a = r.standard_normal((rows, hq, d)).astype(np.float32)
    cache_l = r.standard_normal((rows, hq)).astype(np.float32)
    dec = (r.random((B, hq)) < 0.5).astype(np.uint8)
    dec[0, 0] = 0
    exp_a, exp_l = want_a.copy(), want_l.copy()
    for b in range(B):
        for h in range(hq):
            if dec[b, h]:
                exp_a[b * nb:(b + 1) * nb, h] = cache_a[b * nb:(b + 1) * nb, h]
                exp_l[b * nb:(b + 1) * nb, h] = cache_l[b * nb:(b + 1) * nb, h]
    want_f, want_lf = oracle.merge(exp_a, exp_l, want_ai, want_li)
    q, k, v = dev_in(s.q[0], dtype), dev_in(s.k[0], dtype), dev_in(s.v[0], dtype)
    if lp > 0:
        kp, vp = dev_in(s.kp, dtype), dev_in(s.vp, dtype)
    else:
        kp = vp = torch.zeros(B, hkv, 0, d, device=DEV, dtype=q.dtype)
    ws = torch.zeros(max(1, ba.ba_prefix_attn_workspace(q, kp, vp)), device=DEV, dtype=torch.uint8)
    a_out = torch.from_numpy(cache_a).to(DEV)
    l_out = torch.from_numpy(cache_l).to(DEV)
    a_in = torch.full((rows, hq, d), 3.0, device=DEV)
    l_in = torch.full((rows, hq), 3.0, device=DEV)
    a_full = torch.full((rows, hq, d), 5.0, device=DEV)
    l_full = torch.full((rows, hq), 5.0, device=DEV)
    ba.ba_split_attn(q, kp, vp, k, v, a_out, l_out, a_in, l_in, a_full, l_full, ws,
                     decision=torch.from_numpy(dec).to(DEV))
    torch.cuda.synchronize()
    check_a(host(a_in), want_ai, "A_in")
    check_l(host(l_in), want_li, "L_in")
    ga, gl = host(a_out), host(l_out)
    for b in range(B):
        for h in range(hq):
            sl = slice(b * nb, (b + 1) * nb)
            if dec[b, h]:
                assert np.array_equal(ga[sl, h], cache_a[sl, h]) and np.array_equal(gl[sl, h], cache_l[sl, h])
            else:
                check_a(ga[sl, h], want_a[sl, h], f"A_out b{b} h{h}")
                check_l(gl[sl, h], want_l[sl, h], f"L_out b{b} h{h}")
    check_a(host(a_full), want_f, "A_full")
    check_l(host(l_full), want_lf, "L_full")


GATED_SHAPES = [
    # (B, hq, hkv, d, lp, nb): few rows (two key-waves, split-KV), 128-row
    # tiles (GQA), the alternating 256-row kernel, d = 64 (few rows and the
    # 256-row kernel)
    (2, 8, 8, 128, 512, 32),
    (2, 8, 2, 128, 600, 32),
    (2, 4, 1, 128, 700, 80),
    (2, 4, 4, 64, 300, 20),
    (2, 4, 1, 64, 500, 60),
]


@pytest.mark.parametrize("mode", ["count", "cosine"])
@pytest.mark.parametrize("shape", GATED_SHAPES)
def test_gated_split_attn(mode, shape):
    # The gate in the attention launch (prefix workgroups waiting for their
    # sequence's decisions) gives what the gate followed by the split pass
    # gives: same decisions and M, attention outputs bit for bit.  Three
    # calls in a row (the ready counts must be reset in between): valid
    # cache with mixed decisions, valid cache again, and no valid cache.
    B, hq, hkv, d, lp, nb = shape
    s = _dense_inputs("bf16", B, hq, hkv, d, lp, nb, seed=91)
    rows = B * nb
    q, k, v = dev_in(s.q[0], "bf16"), dev_in(s.k[0], "bf16"), dev_in(s.v[0], "bf16")
    kp, vp = dev_in(s.kp, "bf16"), dev_in(s.vp, "bf16")
    r = np.random.default_rng(5)
    if mode == "count":
        # sequence 0: one changed position (reuse at tau = 4); sequence 1: five
        q_prev, k_prev, v_prev = q.clone(), k.clone(), v.clone()
        q_prev[0, 3] += 1.0
        for pos in (0, 2, 5, 7, nb - 1):
            (k_prev if pos % 2 else v_prev)[1, pos] += 1.0
        gate_kw = dict(tau=4)
        bmode = ba.BA_GATE_COUNT
    else:
        sig = torch.from_numpy(r.uniform(0.01, 0.8, size=(1, 1, hq, 1)).astype(np.float32)).to(DEV)
        q_prev = (q.float() + sig * torch.randn(q.shape, device=DEV)).to(torch.bfloat16)
        k_prev = v_prev = None
        gate_kw = dict(gamma=0.9)
        bmode = ba.BA_GATE_COSINE
    cache_a = torch.from_numpy(r.standard_normal((rows, hq, d)).astype(np.float32)).to(DEV)
    cache_l = torch.from_numpy(r.standard_normal((rows, hq)).astype(np.float32)).to(DEV)
    nws = max(1, ba.ba_prefix_attn_workspace(q, kp, vp))
    gkw = {} if mode == "cosine" else dict(k_cur=k, k_prev=k_prev, v_cur=v, v_prev=v_prev)

    def buffers():
        return dict(a_out=cache_a.clone(), l_out=cache_l.clone(),
                    a_in=torch.full((rows, hq, d), 3.0, device=DEV), l_in=torch.full((rows, hq), 3.0, device=DEV),
                    a_full=torch.full((rows, hq, d), 5.0, device=DEV), l_full=torch.full((rows, hq), 5.0, device=DEV),
                    dec=torch.full((B, hq), 7, device=DEV, dtype=torch.uint8),
                    m=torch.full((B,), -1, device=DEV, dtype=torch.int32),
                    cos=torch.zeros(B, hq, device=DEV, dtype=torch.float64),
                    ws=torch.zeros(nws, device=DEV, dtype=torch.uint8))

    ref, fused = buffers(), buffers()
    gws_ref = torch.zeros(max(1, ba.ba_reuse_gate_workspace(bmode, q, q_prev, **gkw)), device=DEV, dtype=torch.uint8)
    gws = torch.zeros(ba.ba_gated_split_attn_gate_workspace(bmode, q, q_prev, **gkw), device=DEV, dtype=torch.uint8)
    count = mode == "count"
    for call, valid in enumerate((True, True, False)):
        ba.ba_reuse_gate(bmode, q, q_prev, decision=ref["dec"], workspace=gws_ref, cache_valid=valid,
                         m_count=ref["m"] if count else None, cos=None if count else ref["cos"], **gkw, **gate_kw)
        ba.ba_split_attn(q, kp, vp, k, v, ref["a_out"], ref["l_out"], ref["a_in"], ref["l_in"], ref["a_full"],
                         ref["l_full"], ref["ws"], decision=ref["dec"] if valid else None)
        ba.ba_gated_split_attn(bmode, q_prev, kp, vp, k, v, fused["a_out"], fused["l_out"], fused["a_in"],
                               fused["l_in"], fused["a_full"], fused["l_full"], fused["ws"], q=q,
                               decision=fused["dec"], gate_workspace=gws, k_prev=k_prev, v_prev=v_prev,
                               cache_valid=valid, m_count=fused["m"] if count else None,
                               cos=None if count else fused["cos"], **gate_kw)
        torch.cuda.synchronize()
        assert torch.equal(fused["dec"], ref["dec"]), f"call {call}: decisions differ"
        if count:
            assert torch.equal(fused["m"], ref["m"])
            if call == 0:
                assert host(ref["dec"]).tolist() == [[1] * hq, [0] * hq], "schedule should mix reuse and recompute"
        else:
            # the two reductions differ in workgroup size only
            assert np.allclose(host(fused["cos"]), host(ref["cos"]), rtol=0, atol=1e-12)
            if call == 0:
                dv = host(ref["dec"])
                assert 0 < dv.sum() < dv.size, "gamma should mix reuse and recompute"
        for nm in ("a_out", "l_out", "a_in", "l_in", "a_full", "l_full"):
            assert torch.equal(fused[nm], ref[nm]), f"call {call}: {nm} differs"
        gw = host(gws).view(np.int32)
        assert not gw.any(), "gate workspace not left zero (ready counts, tickets or timeouts)"


@pytest.mark.parametrize("mode", ["count", "cosine"])
def test_gated_split_attn_finer_split(mode):
    # With a valid cache the fused step plans its key split for a partly
    # recomputing step, here 16 splits where the split pass takes 8 (eight
    # sequences of 16 rows, 4096 prefix keys).  Decisions and M are the
    # same; recomputed heads match the oracle's prefix attention, reused
    # heads keep the cache bit for bit, and the merged output agrees with
    # the split pass's to the parity bars (the two splits round P
    # differently).
    B, hq, hkv, d, lp, nb = 8, 8, 8, 128, 4096, 16
    s = _dense_inputs("bf16", B, hq, hkv, d, lp, nb, seed=95)
    rows = B * nb
    q, k, v = dev_in(s.q[0], "bf16"), dev_in(s.k[0], "bf16"), dev_in(s.v[0], "bf16")
    kp, vp = dev_in(s.kp, "bf16"), dev_in(s.vp, "bf16")
    r = np.random.default_rng(6)
    if mode == "count":
        q_prev, k_prev, v_prev = q.clone(), k.clone(), v.clone()
        for b in (1, 4, 6):   # these sequences recompute at tau = 4
            for pos in range(5):
                q_prev[b, pos] += 1.0
        gate_kw, bmode, gkw = dict(tau=4), ba.BA_GATE_COUNT, dict(k_cur=k, k_prev=k_prev, v_cur=v, v_prev=v_prev)
    else:
        sig = torch.from_numpy(r.uniform(0.01, 0.8, size=(1, 1, hq, 1)).astype(np.float32)).to(DEV)
        q_prev = (q.float() + sig * torch.randn(q.shape, device=DEV)).to(torch.bfloat16)
        k_prev = v_prev = None
        gate_kw, bmode, gkw = dict(gamma=0.9), ba.BA_GATE_COSINE, {}
    cache_a = torch.from_numpy(r.standard_normal((rows, hq, d)).astype(np.float32)).to(DEV)
    cache_l = torch.from_numpy(r.standard_normal((rows, hq)).astype(np.float32)).to(DEV)
    nws = max(1, ba.ba_prefix_attn_workspace(q, kp, vp))

    def buffers():
        return dict(a_out=cache_a.clone(), l_out=cache_l.clone(), a_in=torch.empty(rows, hq, d, device=DEV),
                    l_in=torch.empty(rows, hq, device=DEV), a_full=torch.empty(rows, hq, d, device=DEV),
                    l_full=torch.empty(rows, hq, device=DEV), dec=torch.empty(B, hq, device=DEV, dtype=torch.uint8),
                    m=torch.empty(B, device=DEV, dtype=torch.int32),
                    cos=torch.empty(B, hq, device=DEV, dtype=torch.float64),
                    ws=torch.zeros(nws, device=DEV, dtype=torch.uint8))

    ref, fused = buffers(), buffers()
    count = mode == "count"
    gws_ref = torch.zeros(max(1, ba.ba_reuse_gate_workspace(bmode, q, q_prev, **gkw)), device=DEV, dtype=torch.uint8)
    gws = torch.zeros(ba.ba_gated_split_attn_gate_workspace(bmode, q, q_prev, **gkw), device=DEV, dtype=torch.uint8)
    ba.ba_reuse_gate(bmode, q, q_prev, decision=ref["dec"], workspace=gws_ref, cache_valid=True,
                     m_count=ref["m"] if count else None, cos=None if count else ref["cos"], **gkw, **gate_kw)
    ba.ba_split_attn(q, kp, vp, k, v, ref["a_out"], ref["l_out"], ref["a_in"], ref["l_in"], ref["a_full"],
                     ref["l_full"], ref["ws"], decision=ref["dec"])
    ba.ba_gated_split_attn(bmode, q_prev, kp, vp, k, v, fused["a_out"], fused["l_out"], fused["a_in"],
                           fused["l_in"], fused["a_full"], fused["l_full"], fused["ws"], q=q, decision=fused["dec"],
                           gate_workspace=gws, k_prev=k_prev, v_prev=v_prev, cache_valid=True,
                           m_count=fused["m"] if count else None, cos=None if count else fused["cos"], **gate_kw)
    torch.cuda.synchronize()
    assert torch.equal(fused["dec"], ref["dec"])
    dv = host(ref["dec"])
    assert 0 < dv.sum() < dv.size, "the decisions should mix reuse and recompute"
    if count:
        assert torch.equal(fused["m"], ref["m"])
    reused = np.repeat(dv.astype(bool), nb, axis=0)   # [rows, hq]
    a_out, l_out = host(fused["a_out"]), host(fused["l_out"])
    assert np.array_equal(a_out[reused], host(cache_a)[reused])
    assert np.array_equal(l_out[reused], host(cache_l)[reused])
    want_a, want_l = _oracle_prefix(s)
    check_a(a_out[~reused], want_a[~reused], "A_out (recomputed heads)")
    check_l(l_out[~reused], want_l[~reused], "L_out (recomputed heads)")
    assert torch.equal(fused["a_in"], ref["a_in"]) and torch.equal(fused["l_in"], ref["l_in"])
    check_a(host(fused["a_full"]), host(ref["a_full"]), "A_full against the split pass")
    check_l(host(fused["l_full"]), host(ref["l_full"]), "L_full against the split pass")
    assert not host(gws).view(np.int32).any(), "gate workspace not left zero"


@pytest.mark.parametrize("lp,hkv,nb", [(512, 8, 32), (64, 8, 32), (1000, 2, 64)])
@pytest.mark.parametrize("mode", ["count", "cosine"])
def test_gated_split_attn_gives_up(mode, lp, hkv, nb):
    # The prefix workgroups' bounded wait for the gate, forced to give up at
    # once from the host (wait_polls < 0): every gated prefix work item is
    # counted and computed into the split workspace, and the combine pass,
    # which runs after the gate, applies the gate's decisions.  So the
    # outputs equal those of the gate followed by the split pass, with
    # several key splits (lp 512) and with one (lp 64), and reused heads keep
    # their cache bit for bit.  256 rows per KV head (hkv 2, nb 64) run the
    # 256-row kernel, whose count-gated steps use persistent prefix
    # workgroups.
    B, hq, d = 2, 8, 128
    s = _dense_inputs("bf16", B, hq, hkv, d, lp, nb, seed=93)
    rows = B * nb
    q, k, v = dev_in(s.q[0], "bf16"), dev_in(s.k[0], "bf16"), dev_in(s.v[0], "bf16")
    kp, vp = dev_in(s.kp, "bf16"), dev_in(s.vp, "bf16")
    nws = ba.ba_prefix_attn_workspace(q, kp, vp)
    assert nws > 0, "a gated fused step always has a split workspace"
    if mode == "count":
        q_prev, k_prev, v_prev = q.clone(), k.clone(), v.clone()
        for pos in range(6):
            q_prev[1, pos] += 1.0        # sequence 0 reused, sequence 1 recomputed
        bmode, gkw, gate_kw = ba.BA_GATE_COUNT, dict(k_cur=k, k_prev=k_prev, v_cur=v, v_prev=v_prev), dict(tau=4)
    else:
        q_prev = (q.float() + 0.3 * torch.randn(q.shape, device=DEV, generator=torch.Generator(DEV).manual_seed(3))
                  ).to(torch.bfloat16)
        k_prev = v_prev = None
        q_prev[0] = q[0]                 # sequence 0 reused (cosine 1)
        bmode, gkw, gate_kw = ba.BA_GATE_COSINE, {}, dict(gamma=0.99)
    r = np.random.default_rng(7)
    cache_a_h = r.standard_normal((rows, hq, d)).astype(np.float32)
    cache_l_h = r.standard_normal((rows, hq)).astype(np.float32)
    cache_a = torch.from_numpy(cache_a_h).to(DEV)
    cache_l = torch.from_numpy(cache_l_h).to(DEV)
    outs = {}
    for which in ("ref", "fused"):
        o = dict(a_out=cache_a.clone(), l_out=cache_l.clone(), a_in=torch.empty(rows, hq, d, device=DEV),
                 l_in=torch.empty(rows, hq, device=DEV), a_full=torch.empty(rows, hq, d, device=DEV),
                 l_full=torch.empty(rows, hq, device=DEV), dec=torch.empty(B, hq, device=DEV, dtype=torch.uint8),
                 m=torch.empty(B, device=DEV, dtype=torch.int32), cos=torch.empty(B, hq, device=DEV, dtype=torch.float64),
                 ws=torch.zeros(nws, device=DEV, dtype=torch.uint8))
        count = mode == "count"
        if which == "ref":
            gws = torch.zeros(max(1, ba.ba_reuse_gate_workspace(bmode, q, q_prev, **gkw)), device=DEV, dtype=torch.uint8)
            ba.ba_reuse_gate(bmode, q, q_prev, decision=o["dec"], workspace=gws, m_count=o["m"] if count else None,
                             cos=None if count else o["cos"], **gkw, **gate_kw)
            ba.ba_split_attn(q, kp, vp, k, v, o["a_out"], o["l_out"], o["a_in"], o["l_in"], o["a_full"], o["l_full"],
                             o["ws"], decision=o["dec"])
        else:
            gws = torch.zeros(ba.ba_gated_split_attn_gate_workspace(bmode, q, q_prev, **gkw), device=DEV,
                              dtype=torch.uint8)
            gave_up = torch.zeros(1, device=DEV, dtype=torch.int32)
            ba.ba_gated_split_attn(bmode, q_prev, kp, vp, k, v, o["a_out"], o["l_out"], o["a_in"], o["l_in"],
                                   o["a_full"], o["l_full"], o["ws"], q=q, decision=o["dec"], gate_workspace=gws,
                                   k_prev=k_prev, v_prev=v_prev, m_count=o["m"] if count else None,
                                   cos=None if count else o["cos"], wait_polls=-1, gave_up=gave_up, **gate_kw)
            o["gws"], o["gave_up"] = gws, gave_up
        torch.cuda.synchronize()
        outs[which] = o
    ref, fused = outs["ref"], outs["fused"]
    dv = host(ref["dec"])
    assert dv[0].all() and not dv[1].any(), "schedule should reuse sequence 0 and recompute sequence 1"
    assert torch.equal(fused["dec"], ref["dec"])
    assert int(fused["gave_up"].item()) > 0, "no prefix workgroup was counted as giving up"
    assert not host(fused["gws"]).view(np.int32).any(), "gate workspace not left zero"
    for nm in ("a_in", "l_in", "a_full", "l_full"):
        assert torch.allclose(fused[nm], ref[nm], rtol=1e-6, atol=1e-6), nm
    # recomputed heads' A_out is fresh either way; reused heads keep the cache
    for nm in ("a_out", "l_out"):
        assert torch.equal(fused[nm][nb:], ref[nm][nb:]), nm
        assert torch.equal(fused[nm][:nb], ref[nm][:nb]), nm
    np.testing.assert_array_equal(host(fused["a_out"])[:nb], cache_a_h[:nb])
    np.testing.assert_array_equal(host(fused["l_out"])[:nb], cache_l_h[:nb])
    # and against the oracle: sequence 1 recomputed with the current Q,
    # sequence 0 merged with its (arbitrary) cache
    wa_in, wl_in = _oracle_block(s)
    wa_out, wl_out = _oracle_prefix(s)
    wa_out[:nb], wl_out[:nb] = cache_a_h[:nb], cache_l_h[:nb]
    wa, wl = oracle.merge(wa_out, wl_out, wa_in, wl_in)
    check_a(host(fused["a_full"]), wa, "A_full against the oracle")
    check_l(host(fused["l_full"]), wl, "L_full against the oracle")


SPARSE_SHAPES = [
    # (B, hq, hkv, d, lp, nb, density): few rows (two key-waves), 128-row
    # tiles (GQA), the alternating 256-row kernel, d = 64; ragged last
    # blocks; enough blocks for several list splits (at most 64 per
    # workgroup); every block listed
    (2, 4, 4, 128, 64 * 40 + 17, 32, 0.3),
    (1, 8, 2, 128, 64 * 150, 32, 1.0),
    (1, 4, 1, 128, 64 * 20 + 1, 80, 0.25),
    (2, 4, 4, 64, 64 * 9 + 40, 20, 0.5),
]


@pytest.mark.parametrize("shape", SPARSE_SHAPES)
def test_sparse_prefix_attn(shape):
    # Prefix attention over a key-block list and over its complement, each
    # against the oracle on every row, and their merge against attention
    # over the whole prefix (the residual-reuse identity).
    B, hq, hkv, d, lp, nb, dens = shape
    s = _dense_inputs("bf16", B, hq, hkv, d, lp, nb, seed=95)
    sel, rest = make_key_block_lists(B=B, hkv=hkv, lp=lp, density=dens, seed=4)
    q, kp, vp = dev_in(s.q[0], "bf16"), dev_in(s.kp, "bf16"), dev_in(s.vp, "bf16")
    rows = B * nb
    g = hq // hkv
    got = {}
    for nm, lst in (("sel", sel), ("rest", rest)):
        bl = torch.from_numpy(np.ascontiguousarray(lst)).to(DEV)
        ws = torch.zeros(max(1, ba.ba_sparse_prefix_attn_workspace(q, kp, vp, bl)), device=DEV, dtype=torch.uint8)
        a = torch.full((rows, hq, d), 777.0, device=DEV)
        l = torch.full((rows, hq), 777.0, device=DEV)
        ba.ba_sparse_prefix_attn(q, kp, vp, bl, a, l, ws)
        torch.cuda.synchronize()
        got[nm] = (host(a), host(l))
        want_a = np.zeros((B, nb, hq, d)); want_l = np.zeros((B, nb, hq))
        for b in range(B):
            for h in range(hq):
                want_a[b, :, h], want_l[b, :, h] = oracle.prefix_rows_in_blocks(s, 0, b, h, lst[b, h // g])
        if lst.shape[2] == 0:
            assert np.all(got[nm][0] == 0) and np.all(np.isneginf(got[nm][1]))
        else:
            check_a(got[nm][0], want_a.reshape(rows, hq, d), f"A {nm}")
            check_l(got[nm][1], want_l.reshape(rows, hq), f"L {nm}")
    am, lm = oracle.merge(got["sel"][0].astype(np.float64), got["sel"][1].astype(np.float64),
                          got["rest"][0].astype(np.float64), got["rest"][1].astype(np.float64))
    full_a, full_l = _oracle_prefix(s)
    check_a(am, full_a, "A merged")
    check_l(lm, full_l, "L merged")


def test_sparse_prefix_attn_gated_and_empty():
    # The decision gates a listed pass like the dense one (reused heads keep
    # the cache), and an empty list gives A = 0, L = -inf.
    B, hq, hkv, d, lp, nb = 2, 4, 4, 128, 64 * 12, 32
    s = _dense_inputs("bf16", B, hq, hkv, d, lp, nb, seed=96)
    sel, _ = make_key_block_lists(B=B, hkv=hkv, lp=lp, density=0.5, seed=6)
    q, kp, vp = dev_in(s.q[0], "bf16"), dev_in(s.kp, "bf16"), dev_in(s.vp, "bf16")
    rows = B * nb
    dec = np.array([[1, 0, 1, 0], [0, 0, 1, 1]], dtype=np.uint8)
    r = np.random.default_rng(3)
    cache_a = r.standard_normal((rows, hq, d)).astype(np.float32)
    cache_l = r.standard_normal((rows, hq)).astype(np.float32)
    a = torch.from_numpy(cache_a).to(DEV)
    l = torch.from_numpy(cache_l).to(DEV)
    bl = torch.from_numpy(sel).to(DEV)
    ws = torch.zeros(max(1, ba.ba_sparse_prefix_attn_workspace(q, kp, vp, bl)), device=DEV, dtype=torch.uint8)
    ba.ba_sparse_prefix_attn(q, kp, vp, bl, a, l, ws, decision=torch.from_numpy(dec).to(DEV))
    torch.cuda.synchronize()
    ga, gl = host(a), host(l)
    for b in range(B):
        for h in range(hq):
            sl = slice(b * nb, (b + 1) * nb)
            if dec[b, h]:
                assert np.array_equal(ga[sl, h], cache_a[sl, h]) and np.array_equal(gl[sl, h], cache_l[sl, h])
            else:
                wa, wl = oracle.prefix_rows_in_blocks(s, 0, b, h, sel[b, h])
                check_a(ga[sl, h], wa, f"A b{b} h{h}")
                check_l(gl[sl, h], wl, f"L b{b} h{h}")
    empty = torch.zeros(B, hkv, 0, device=DEV, dtype=torch.int32)
    a0 = torch.full((rows, hq, d), 5.0, device=DEV)
    l0 = torch.full((rows, hq), 5.0, device=DEV)
    ws0 = torch.zeros(max(1, ba.ba_sparse_prefix_attn_workspace(q, kp, vp, empty)), device=DEV, dtype=torch.uint8)
    ba.ba_sparse_prefix_attn(q, kp, vp, empty, a0, l0, ws0)
    torch.cuda.synchronize()
    assert torch.all(a0 == 0) and torch.all(torch.isneginf(l0))


KL_SHAPES = [
    # (n rows, vocab, dtype, extra row padding): vector loads with and
    # without a ragged tail, float32, a large vocabulary, and rows whose
    # stride breaks 16-byte alignment (scalar loads)
    (37, 1000, "bf16", 0),
    (64, 4099, "bf16", 0),
    (16, 2050, "f32", 0),
    (5, 126464, "bf16", 0),
    (9, 777, "bf16", 3),
]


@pytest.mark.parametrize("shape", KL_SHAPES)
def test_kl_lock(shape):
    # KL of each row's current posterior from the previous step's against the
    # oracle, and the lock update (eligible rows below eps lock; locks stay).
    n, vocab, dtype, pad = shape
    cur, prev, _ = make_logit_pair(n=n, vocab=vocab, dtype=dtype, seed=n + vocab)
    want = oracle.kl_rows(oracle.to_f64(cur, dtype), oracle.to_f64(prev, dtype))

    def dev(x):
        t = dev_in(x, dtype)
        if pad:
            big = torch.zeros(n, vocab + pad, device=DEV, dtype=t.dtype)
            big[:, :vocab] = t
            return big[:, :vocab]
        return t

    xc, xp = dev(cur), dev(prev)
    eps = float(np.median(want))
    r = np.random.default_rng(n)
    eligible = (r.random(n) < 0.8).astype(np.uint8)
    locked0 = (r.random(n) < 0.2).astype(np.uint8)
    kl = torch.full((n,), -1.0, device=DEV)
    locked = torch.from_numpy(locked0.copy()).to(DEV)
    ba.ba_kl_lock(xc, xp, eps=eps, kl=kl, locked=locked, eligible=torch.from_numpy(eligible).to(DEV))
    torch.cuda.synchronize()
    got = host(kl).astype(np.float64)
    tol = 2e-6 + 1e-5 * want
    bad = np.abs(got - want) > tol
    assert not bad.any(), f"KL off at rows {np.flatnonzero(bad)[:5]}: {got[bad][:5]} vs {want[bad][:5]}"
    exp_lock = oracle.lock_update(locked0, eligible, want, eps)
    gl = host(locked)
    near = np.abs(want - eps) <= tol
    assert np.array_equal(gl[~near], exp_lock[~near])
    assert near.sum() <= 1   # the median row itself may sit on the threshold


def test_kl_lock_edge_values():
    # -inf logits (zero-probability entries), a q with zero mass where p has
    # some (KL = +inf: never locks), identical rows (KL = 0), and kl-only /
    # lock-only calls.
    vocab = 300
    cur, prev, _ = make_logit_pair(n=4, vocab=vocab, dtype="f32", seed=8)
    cur = cur.copy(); prev = prev.copy()
    cur[0, :50] = -np.inf; prev[0, :50] = -np.inf
    prev[1, 7] = -np.inf
    prev[2] = cur[2]
    cur[3, 100:] = -np.inf
    want = oracle.kl_rows(cur, prev)
    assert np.isinf(want[1]) and want[2] == 0
    xc, xp = torch.from_numpy(cur).to(DEV), torch.from_numpy(prev).to(DEV)
    kl = torch.empty(4, device=DEV)
    ba.ba_kl_lock(xc, xp, eps=1e-3, kl=kl)
    locked = torch.zeros(4, device=DEV, dtype=torch.uint8)
    ba.ba_kl_lock(xc, xp, eps=1e-3, locked=locked)
    torch.cuda.synchronize()
    got = host(kl).astype(np.float64)
    assert np.isinf(got[1]) and got[2] == 0
    for r_ in (0, 3):
        assert abs(got[r_] - want[r_]) <= 2e-6 + 1e-5 * want[r_]
    assert host(locked).tolist() == [int(want[0] < 1e-3), 0, 1, int(want[3] < 1e-3)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kl_lock_shift_paths(dtype):
    # Rows that move a thread's shift after its first chunk or need the
    # guarded step: a rising ramp over 120 nats (the maximum arrives last),
    # a falling one, a late spike far above the rest, a leading run of -inf
    # in both rows, -inf runs in one row only, and logits near the float32
    # exponential's range; vocabulary with a ragged tail.
    vocab = 8 * 1024 + 5
    r = np.random.default_rng(11)
    cur = r.normal(0.0, 3.0, (8, vocab))
    prev = cur + r.normal(0.0, 0.05, (8, vocab))
    ramp = np.linspace(-60.0, 60.0, vocab)
    cur[0] = ramp + r.normal(0.0, 0.5, vocab)
    prev[0] = ramp + r.normal(0.0, 0.5, vocab)
    cur[1] = ramp[::-1] + r.normal(0.0, 0.5, vocab)
    prev[1] = ramp[::-1] + r.normal(0.0, 0.5, vocab)
    cur[2, vocab - 700] += 90.0
    prev[2, vocab - 650] += 88.0
    cur[3, :3000] = -np.inf
    prev[3, :3000] = -np.inf
    cur[4, 100:5000:3] = -np.inf
    cur[5] += 75.0
    prev[5] += 70.0
    cur[6] *= 12.0
    prev[6] *= 12.0
    if dtype == "bf16":
        # (round to nearest even keeps the -inf bit patterns)
        cur, prev = round_to_bf16_bits(cur.astype(np.float32)), round_to_bf16_bits(prev.astype(np.float32))
    else:
        cur, prev = cur.astype(np.float32), prev.astype(np.float32)
    want = oracle.kl_rows(oracle.to_f64(cur, dtype), oracle.to_f64(prev, dtype))
    assert np.all(np.isfinite(want))
    kl = torch.full((8,), -1.0, device=DEV)
    ba.ba_kl_lock(dev_in(cur, dtype), dev_in(prev, dtype), eps=1e-3, kl=kl)
    torch.cuda.synchronize()
    got = host(kl).astype(np.float64)
    tol = 2e-6 + 1e-5 * want
    bad = np.abs(got - want) > tol
    assert not bad.any(), f"KL off at rows {np.flatnonzero(bad)}: {got[bad]} vs {want[bad]}"


def test_split_attn_varlen():
    # Branches of different block sizes and prefix lengths (one prefix
    # empty), locked positions packed out, in one varlen split-attention call.
    vb = make_varlen_batch(block_sizes=(3, 16, 40, 7), prefix_lens=(100, 0, 700, 333), h=4, d=128,
                           lock_p=0.3, seed=21)
    ref = oracle.run_varlen(vb)
    n = int(vb.block_sizes.sum())
    nbr = vb.block_sizes.size
    cu_q = torch.empty(nbr + 1, device=DEV, dtype=torch.int32)
    gather = torch.empty(n, device=DEV, dtype=torch.int32)
    total = torch.empty(1, device=DEV, dtype=torch.int32)
    qp = torch.zeros(n, vb.h, vb.d, device=DEV, dtype=torch.bfloat16)
    ba.ba_varlen_pack(vb.block_sizes, torch.from_numpy(vb.locked).to(DEV), cu_q, gather, total, dev_bits(vb.q), qp)
    cu_kp = torch.from_numpy(np.concatenate([[0], np.cumsum(vb.prefix_lens)]).astype(np.int32)).to(DEV)
    cu_kb = torch.from_numpy(np.concatenate([[0], np.cumsum(vb.block_sizes)]).astype(np.int32)).to(DEV)
    kp, vp = dev_bits(vb.kp), dev_bits(vb.vp)
    kb, vbk = dev_bits(vb.k), dev_bits(vb.v)
    max_q = int(vb.block_sizes.max())
    outs = {nm: torch.full((n, vb.h, vb.d), 7.0, device=DEV) for nm in ("a_out", "a_in", "a_full")}
    outs.update({nm: torch.full((n, vb.h), 7.0, device=DEV) for nm in ("l_out", "l_in", "l_full")})
    ws = torch.zeros(max(1, ba.ba_prefix_attn_workspace(qp, kp, vp, q_layout="thd", kv_layout="htd", cu_q=cu_q,
                                                        cu_k=cu_kp, max_q=max_q, max_k=int(vb.prefix_lens.max()))),
                     device=DEV, dtype=torch.uint8)
    ba.ba_split_attn(qp, kp, vp, kb, vbk, outs["a_out"], outs["l_out"], outs["a_in"], outs["l_in"],
                     outs["a_full"], outs["l_full"], ws, q_layout="thd", kv_layout="htd", block_kv_layout="thd",
                     cu_q=cu_q, cu_kp=cu_kp, cu_k=cu_kb, max_q=max_q, max_kp=int(vb.prefix_lens.max()),
                     max_k=int(vb.block_sizes.max()))
    torch.cuda.synchronize()
    tot = ref["total"]
    assert int(total.item()) == tot
    for nm in ("a_out", "a_in", "a_full"):
        check_a(host(outs[nm])[:tot], ref[nm], nm)
    for nm in ("l_out", "l_in", "l_full"):
        check_l(host(outs[nm])[:tot], ref[nm], nm)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("nb", [20, 150])
def test_prefix_attn_empty_prefix(dtype, nb):
    # nb = 150: 300 rows per KV head, the 256-row kernel
    s = _dense_inputs(dtype, 2, 4, 2, 128, 0, nb, seed=62)
    q = dev_in(s.q[0], dtype)
    kp = torch.zeros(2, 2, 0, 128, device=DEV, dtype=q.dtype)
    a = torch.full((2 * nb, 4, 128), 5.0, device=DEV)
    l = torch.full((2 * nb, 4), 5.0, device=DEV)
    assert ba.ba_prefix_attn_workspace(q, kp, kp) == 0
    ba.ba_prefix_attn(q, kp, kp, a, l)
    torch.cuda.synchronize()
    assert torch.all(a == 0) and torch.all(torch.isneginf(l))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefix_attn_bshd_layout(dtype):
    s = _dense_inputs(dtype, 2, 4, 2, 128, 700, 30, seed=63)
    want_a, want_l = _oracle_prefix(s)
    q = dev_in(s.q[0], dtype)
    kp = dev_in(s.kp, dtype).transpose(1, 2).contiguous()  # [B, Lp, Hkv, d]
    vp = dev_in(s.vp, dtype).transpose(1, 2).contiguous()
    ws = torch.zeros(max(1, ba.ba_prefix_attn_workspace(q, kp, vp, kv_layout="bshd")), device=DEV,
                     dtype=torch.uint8)
    a = torch.empty(60, 4, 128, device=DEV)
    l = torch.empty(60, 4, device=DEV)
    ba.ba_prefix_attn(q, kp, vp, a, l, ws, kv_layout="bshd")
    torch.cuda.synchronize()
    check_a(host(a), want_a, "A_out")
    check_l(host(l), want_l, "L_out")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", DENSE_SHAPES)
def test_block_attn_fused_merge(dtype, shape):
    B, hq, hkv, d, lp, nb = shape
    _check_block_attn(dtype, B, hq, hkv, d, nb, seed=hash(shape) % 997)


# Blocks of more than 192 rows per KV head and more than 512 keys (the
# alternating 256-row kernel): GQA with a ragged row tile and key tile, a
# video-like pair of heads (1560 rows and keys: 6 full row tiles, a 24-row
# tail, 24 full key tiles and a 24-key tail), d = 64 with two sequences.
BIG_BLOCK_SHAPES = [
    (1, 4, 1, 128, 600),
    (1, 2, 2, 128, 1560),
    (2, 2, 1, 64, 530),
]


@pytest.mark.parametrize("shape", BIG_BLOCK_SHAPES)
def test_block_attn_many_rows_and_keys(shape):
    B, hq, hkv, d, nb = shape
    _check_block_attn("bf16", B, hq, hkv, d, nb, seed=nb)


def _check_block_attn(dtype, B, hq, hkv, d, nb, seed):
    # A_in/L_in against the in-block oracle, A_full/L_full against its merge
    # with a random cache (some cached rows empty: L = -inf); a call without
    # A_in/L_in gives the same A_full bit for bit, and one without the cache
    # the same A_in/L_in.
    s = _dense_inputs(dtype, B, hq, hkv, d, 4, nb, seed=seed)
    want_a, want_l = _oracle_block(s)
    r = np.random.default_rng(5)
    rows = B * nb
    ac = r.standard_normal((rows, hq, d)).astype(np.float32)
    lc = (r.standard_normal((rows, hq)) * 3 + 2).astype(np.float32)
    lc[::5, 0] = -np.inf
    ac[::5, 0] = 0.0
    wf, wlf = oracle.merge(ac, lc, want_a, want_l)
    q, k, v = dev_in(s.q[0], dtype), dev_in(s.k[0], dtype), dev_in(s.v[0], dtype)
    outs = [torch.full((rows, hq, d), 9.0, device=DEV), torch.full((rows, hq), 9.0, device=DEV),
            torch.full((rows, hq, d), 9.0, device=DEV), torch.full((rows, hq), 9.0, device=DEV)]
    ba.ba_block_attn(q, k, v, a_cache=dev_f32(ac), l_cache=dev_f32(lc), a_in=outs[0], l_in=outs[1],
                     a_full=outs[2], l_full=outs[3])
    torch.cuda.synchronize()
    check_a(host(outs[0]), want_a, "A_in")
    check_l(host(outs[1]), want_l, "L_in")
    check_a(host(outs[2]), wf, "A_full")
    check_l(host(outs[3]), wlf, "L_full")
    # only the merged output
    af = torch.zeros(rows, hq, d, device=DEV)
    ba.ba_block_attn(q, k, v, a_cache=dev_f32(ac), l_cache=dev_f32(lc), a_full=af)
    torch.cuda.synchronize()
    assert torch.equal(af, outs[2])
    # no cache: the in-block part alone
    ai, li = torch.zeros(rows, hq, d, device=DEV), torch.zeros(rows, hq, device=DEV)
    ba.ba_block_attn(q, k, v, a_in=ai, l_in=li)
    torch.cuda.synchronize()
    assert torch.equal(ai, outs[0]) and torch.equal(li, outs[1])


def test_block_attn_guard_bands():
    s = _dense_inputs("bf16", 2, 4, 2, 128, 4, 37, seed=64)
    q, k, v = dev_bits(s.q[0]), dev_bits(s.k[0]), dev_bits(s.v[0])
    rows = 74
    pad = 4096
    buf = torch.full((pad + rows * 4 * 128 + pad,), 31.0, device=DEV)
    lbuf = torch.full((pad + rows * 4 + pad,), 31.0, device=DEV)
    a = buf[pad:pad + rows * 4 * 128].view(rows, 4, 128)
    l = lbuf[pad:pad + rows * 4].view(rows, 4)
    ba.ba_block_attn(q, k, v, a_in=a, l_in=l)
    kp, vp = dev_bits(s.kp), dev_bits(s.vp)
    ba.ba_prefix_attn(q, kp, vp, a, l)
    torch.cuda.synchronize()
    assert torch.all(buf[:pad] == 31.0) and torch.all(buf[pad + rows * 512:] == 31.0)
    assert torch.all(lbuf[:pad] == 31.0) and torch.all(lbuf[pad + rows * 4:] == 31.0)


def test_nan_poisoned_cache():
    """Reuse really reads the cache (NaN shows up); recompute really
    overwrites it (NaN gone)."""
    s = make_block_schedule(dtype="bf16", B=1, hq=4, hkv=4, d=128, lp=300, nb=16, steps=2,
                            schedule="none", gate="count", tau=4, seed=65)
    kp, vp = dev_bits(s.kp), dev_bits(s.vp)
    q = [dev_bits(x) for x in s.q]
    k = [dev_bits(x) for x in s.k]
    v = [dev_bits(x) for x in s.v]
    attn = ba.CachedBlockAttention(kp, vp, nb=16, hq=4, gate="count", tau=4)
    attn.step(q[1], k[1], v[1], q[0], k[0], v[0])
    attn.a_out.fill_(float("nan"))
    attn.l_out.fill_(float("nan"))
    af, _ = attn.step(q[2], k[2], v[2], q[1], k[1], v[1])   # unchanged block: reuse
    torch.cuda.synchronize()
    assert int(attn.decision.min()) == 1
    assert torch.isnan(af).all()
    attn.start_block()
    af, _ = attn.step(q[2], k[2], v[2], q[1], k[1], v[1])   # invalid cache: recompute
    torch.cuda.synchronize()
    assert int(attn.decision.max()) == 0
    assert torch.isfinite(af).all()


# ----------------------------------------------------------------------------
# varlen
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("d", [128, 64])
def test_varlen_attention(d):
    vb = make_varlen_batch(block_sizes=(3, 0, 5, 8, 33, 70), prefix_lens=(100, 40, 0, 70, 300, 1111),
                           h=4, d=d, lock_p=0.3, seed=66)
    ref = oracle.run_varlen(vb)
    n = int(vb.block_sizes.sum())
    nbr = vb.block_sizes.size
    locked = torch.from_numpy(vb.locked).to(DEV)
    cu_q = torch.empty(nbr + 1, device=DEV, dtype=torch.int32)
    gather = torch.empty(n, device=DEV, dtype=torch.int32)
    total = torch.empty(1, device=DEV, dtype=torch.int32)
    qsrc = dev_bits(vb.q)
    qp = torch.zeros(n, vb.h, d, device=DEV, dtype=torch.bfloat16)
    ba.ba_varlen_pack(vb.block_sizes, locked, cu_q, gather, total, qsrc, qp)
    cu_kp = torch.from_numpy(np.concatenate([[0], np.cumsum(vb.prefix_lens)]).astype(np.int32)).to(DEV)
    cu_kb = torch.from_numpy(np.concatenate([[0], np.cumsum(vb.block_sizes)]).astype(np.int32)).to(DEV)
    kp, vp = dev_bits(vb.kp), dev_bits(vb.vp)          # [H, sum L, d]
    kb, vbk = dev_bits(vb.k), dev_bits(vb.v)           # [sum B, H, d]
    max_q = int(vb.block_sizes.max())
    a_out = torch.full((n, vb.h, d), 3.0, device=DEV)
    l_out = torch.full((n, vb.h), 3.0, device=DEV)
    kw = dict(q_layout="thd", cu_q=cu_q, max_q=max_q)
    ws = torch.zeros(max(1, ba.ba_prefix_attn_workspace(qp, kp, vp, kv_layout="htd", cu_k=cu_kp,
                                                         max_k=int(vb.prefix_lens.max()), **kw)),
                     device=DEV, dtype=torch.uint8)
    ba.ba_prefix_attn(qp, kp, vp, a_out, l_out, ws, kv_layout="htd", cu_k=cu_kp,
                      max_k=int(vb.prefix_lens.max()), **kw)
    a_full = torch.full((n, vb.h, d), 3.0, device=DEV)
    l_full = torch.full((n, vb.h), 3.0, device=DEV)
    a_in = torch.full((n, vb.h, d), 3.0, device=DEV)
    ba.ba_block_attn(qp, kb, vbk, a_cache=a_out, l_cache=l_out, a_in=a_in, a_full=a_full, l_full=l_full,
                     kv_layout="thd", cu_k=cu_kb, max_k=int(vb.block_sizes.max()), **kw)
    torch.cuda.synchronize()
    tot = ref["total"]
    assert int(total.item()) == tot
    assert cu_q.cpu().numpy().tolist() == ref["cu_seqlens"].tolist()
    check_a(host(a_out)[:tot], ref["a_out"], "A_out varlen")
    check_l(host(l_out)[:tot], ref["l_out"], "L_out varlen")
    check_a(host(a_in)[:tot], ref["a_in"], "A_in varlen")
    check_a(host(a_full)[:tot], ref["a_full"], "A_full varlen")
    check_l(host(l_full)[:tot], ref["l_full"], "L_full varlen")
    # rows past the packed total are never written
    assert torch.all(a_full[tot:] == 3.0) and torch.all(a_out[tot:] == 3.0)


def test_varlen_gqa_256_row_kernel():
    # Packed (thd) query rows of a GQA batch with more than 192 rows per KV
    # head, so the prefix part and (with more than 512 block keys) the
    # in-block part run on the alternating 256-row kernel with packed Q and
    # packed K/V: blocks of 530, 0 and 201 positions, prefixes of 300, 50 and
    # 700 keys, 8 query heads on 2 KV heads.
    rng = np.random.default_rng(77)
    hq, hkv, d = 8, 2, 128
    g = hq // hkv
    nq = np.array([530, 0, 201])
    lp = np.array([300, 50, 700])
    n, nl = int(nq.sum()), int(lp.sum())
    scale = 1.0 / math.sqrt(d)

    def draw(*shape):
        return round_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))

    q, kb, vb = draw(n, hq, d), draw(n, hkv, d), draw(n, hkv, d)
    kp, vp = draw(nl, hkv, d), draw(nl, hkv, d)
    cq = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lp)]).astype(np.int32)
    want = {nm: np.zeros((n, hq, d)) for nm in ("a_out", "a_in", "a_full")}
    want.update({nm: np.zeros((n, hq)) for nm in ("l_out", "l_in", "l_full")})
    f = lambda x: oracle.to_f64(x, "bf16")
    for b in range(nq.size):
        r = slice(cq[b], cq[b + 1])
        for h in range(hq):
            qq = f(q[r, h])
            ao, lo = oracle.attention(qq, f(kp[ck[b]:ck[b + 1], h // g]), f(vp[ck[b]:ck[b + 1], h // g]), scale)
            ai, li = oracle.attention(qq, f(kb[r, h // g]), f(vb[r, h // g]), scale)
            af, lf = oracle.merge(ao, lo, ai, li)
            for nm, x in (("a_out", ao), ("l_out", lo), ("a_in", ai), ("l_in", li), ("a_full", af), ("l_full", lf)):
                want[nm][r, h] = x
    cu_q, cu_kp = torch.from_numpy(cq).to(DEV), torch.from_numpy(ck).to(DEV)
    kw = dict(q_layout="thd", cu_q=cu_q, max_q=int(nq.max()))
    pk = dict(kv_layout="thd", cu_k=cu_kp, max_k=int(lp.max()))
    qd = dev_bits(q)
    out = {nm: torch.full((n, hq, d), 3.0, device=DEV) for nm in ("a_out", "a_in", "a_full")}
    out.update({nm: torch.full((n, hq), 3.0, device=DEV) for nm in ("l_out", "l_in", "l_full")})
    ws = torch.zeros(max(1, ba.ba_prefix_attn_workspace(qd, dev_bits(kp), dev_bits(vp), **pk, **kw)), device=DEV,
                     dtype=torch.uint8)
    ba.ba_prefix_attn(qd, dev_bits(kp), dev_bits(vp), out["a_out"], out["l_out"], ws, **pk, **kw)
    ba.ba_block_attn(qd, dev_bits(kb), dev_bits(vb), a_cache=out["a_out"], l_cache=out["l_out"], a_in=out["a_in"],
                     l_in=out["l_in"], a_full=out["a_full"], l_full=out["l_full"], kv_layout="thd", cu_k=cu_q,
                     max_k=int(nq.max()), **kw)
    torch.cuda.synchronize()
    for nm in ("a_out", "a_in", "a_full"):
        check_a(host(out[nm]), want[nm], nm)
    for nm in ("l_out", "l_in", "l_full"):
        check_l(host(out[nm]), want[nm], nm)


# ----------------------------------------------------------------------------
# whole schedules through the step driver
# ----------------------------------------------------------------------------

def _run_schedule(s, check_rows=None):
    ref = oracle.run_block(s)
    kp, vp = dev_in(s.kp, s.dtype), dev_in(s.vp, s.dtype)
    q = [dev_in(x, s.dtype) for x in s.q]
    k = [dev_in(x, s.dtype) for x in s.k]
    v = [dev_in(x, s.dtype) for x in s.v]
    attn = ba.CachedBlockAttention(kp, vp, nb=s.nb, hq=s.hq, gate=s.gate, tau=s.tau, gamma=s.gamma,
                                   scale=s.scale)
    reuse_seen = 0
    for t in range(1, s.steps + 1):
        af, lf = attn.step(q[t], k[t], v[t], q[t - 1], k[t - 1], v[t - 1])
        torch.cuda.synchronize()
        dec = attn.decision.cpu().numpy()
        assert np.array_equal(dec, ref[t]["gate"]["decision"]), t
        reuse_seen += int(dec.sum())
        check_a(host(af), ref[t]["a_full"], f"A_full step {t}")
        check_l(host(lf), ref[t]["l_full"], f"L_full step {t}")
        check_a(host(attn.a_out), ref[t]["a_out"], f"A_out cache step {t}")
    return reuse_seen


def test_schedule_tiny_f32():
    """The single-layer float32 workload: 4 heads, d = 64, prefix 256, block
    32, 8 steps redrawing 1-4 rows, tau = 4."""
    from workloads import preset
    s = preset("c1_tiny_f32")
    assert _run_schedule(s) > 0


@pytest.mark.parametrize("schedule,gate", [("redraw", "count"), ("poisson", "count"), ("qnoise", "cosine")])
def test_schedule_bf16(schedule, gate):
    s = make_block_schedule(dtype="bf16", B=2, hq=4, hkv=2, d=128, lp=640, nb=40, steps=6, std=1.0,
                            schedule=schedule, redraw_range=(0, 3), poisson_lam=1.5,
                            sigma_range=(0.01, 0.5), gate=gate, tau=3, gamma=0.95, seed=67)
    assert _run_schedule(s) > 0


@pytest.mark.parametrize("gate,hkv,nb", [
    ("count", 2, 33),     # 128-row tiles: gate, attention launch, then the combine pass
    ("count", 1, 80),     # 256-row kernel, one launch per step (persistent prefix part)
    ("cosine", 1, 80),    # 256-row kernel, one launch per step
])
def test_graph_replay_matches_eager(gate, hkv, nb):
    """A captured block schedule replays to the eager result, every time,
    with eager work and synchronisations between the replays (the launches'
    synchronisation words must be left cleared for the next replay)."""
    s = make_block_schedule(dtype="bf16", B=2, hq=4, hkv=hkv, d=128, lp=900, nb=nb, steps=4, std=1.0,
                            schedule="redraw", redraw_range=(0, 3), sigma_range=(0.01, 0.5), gate=gate, tau=2,
                            gamma=0.95, seed=68)
    kp, vp = dev_bits(s.kp), dev_bits(s.vp)
    q = [dev_bits(x) for x in s.q]
    k = [dev_bits(x) for x in s.k]
    v = [dev_bits(x) for x in s.v]
    eager = ba.CachedBlockAttention(kp, vp, nb=s.nb, hq=s.hq, gate=gate, tau=s.tau, gamma=s.gamma)
    outs = []
    for t in range(1, s.steps + 1):
        af, lf = eager.step(q[t], k[t], v[t], q[t - 1], k[t - 1], v[t - 1])
        outs.append((af.clone(), lf.clone(), eager.a_out.clone(), eager.decision.clone()))
    torch.cuda.synchronize()
    attn = ba.CachedBlockAttention(kp, vp, nb=s.nb, hq=s.hq, gate=gate, tau=s.tau, gamma=s.gamma)
    g = attn.capture_block(q, k, v)
    g1 = attn.capture(q, k, v, [s.steps], new_block=False)
    for rep in range(3):
        attn.a_full.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(attn.a_full, outs[-1][0]) and torch.equal(attn.l_full, outs[-1][1]), rep
        assert torch.equal(attn.a_out, outs[-1][2]) and torch.equal(attn.decision, outs[-1][3]), rep
        junk = torch.randn(1000, device=DEV).sum()  # eager work between replays
        torch.cuda.synchronize()
        del junk
        g1.replay()   # the last step alone, cache valid
        torch.cuda.synchronize()
        assert torch.equal(attn.a_full, outs[-1][0]), rep
