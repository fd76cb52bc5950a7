"""Checks that pin the CPU oracle to facts outside itself.

Each check takes the functions under test as arguments and raises
AssertionError on the first disagreement, so the same checks run against the
oracle (they must pass) and against copies of it with a planted mistake
(they must fail; see test_oracle_mutants.py).

What pins what:
  attention  - mpmath brute force at 50 digits (sum of exp(z_j) v_j over sum
               of exp(z_j), no max shift) on tiny non-square shapes;
               closed forms (one key; identical keys; constant values;
               zero query; shifted keys; empty key set).
  merge      - the split identity: merging attention over two disjoint key
               sets equals attention over their union (to 1e-12); three-way
               associativity and commutativity; the empty set is neutral;
               a set merged with itself; hand-derived worked examples.
  gates      - integer counts against the generator's own record of which
               rows it rewrote and against a pure-Python element loop; the
               strict inequalities at the tau and gamma boundaries with exact
               ties (cos = 24/25); first step recomputes.
  packing    - prefix-sum closed form, ordering, coverage and a round trip.
"""

from __future__ import annotations

import json
import math
import os

import mpmath
import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(x, y, tol, what):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    assert x.shape == y.shape, f"{what}: shape {x.shape} vs {y.shape}"
    both_inf = np.isinf(x) & np.isinf(y) & (np.sign(x) == np.sign(y))
    err = np.where(both_inf, 0.0, np.abs(x - y))
    assert np.all(np.isfinite(err)), f"{what}: non-finite mismatch {x} vs {y}"
    assert err.max(initial=0.0) <= tol, f"{what}: max err {err.max()} > {tol}"


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------

def brute_force_attention(q, k, v, scale, dps=50):
    """Direct high-precision definition, no max shift."""
    with mpmath.workdps(dps):
        n, m = q.shape[0], k.shape[0]
        a = np.zeros((n, v.shape[1]))
        lse = np.zeros(n)
        for i in range(n):
            w = [mpmath.exp(mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[i, c]) * mpmath.mpf(k[j, c])
                                                          for c in range(q.shape[1])))
                 for j in range(m)]
            z = mpmath.fsum(w)
            for c in range(v.shape[1]):
                a[i, c] = float(mpmath.fsum(w[j] * mpmath.mpf(v[j, c]) for j in range(m)) / z)
            lse[i] = float(mpmath.log(z))
        return a, lse


def check_attention(attention):
    rng = np.random.default_rng(7)
    # brute force on tiny, deliberately non-square shapes (n, m, d, dv)
    for (n, m, d, dv, sc) in [(1, 1, 1, 1, 1.0), (2, 3, 2, 3, 0.7), (4, 6, 4, 2, 0.5),
                              (3, 5, 3, 4, 1.3), (4, 2, 4, 5, 0.25)]:
        q = rng.standard_normal((n, d))
        k = rng.standard_normal((m, d))
        v = rng.standard_normal((m, dv))
        a, l = attention(q, k, v, sc)
        ba, bl = brute_force_attention(q, k, v, sc)
        _close(a, ba, 1e-13, f"brute force A {(n, m, d, dv)}")
        _close(l, bl, 1e-13, f"brute force L {(n, m, d, dv)}")
    # large-magnitude scores: the exact definition still holds
    q = rng.standard_normal((2, 3)) * 30
    k = rng.standard_normal((4, 3)) * 30
    v = rng.standard_normal((4, 2))
    a, l = attention(q, k, v, 1.0)
    ba, bl = brute_force_attention(q, k, v, 1.0, dps=80)
    _close(a, ba, 1e-12, "brute force A, large scores")
    _close(l / np.abs(bl), bl / np.abs(bl), 1e-14, "brute force L, large scores")

    d = 5
    q = rng.standard_normal((3, d))
    kk = rng.standard_normal((1, d))
    vv = rng.standard_normal((1, 4))
    a, l = attention(q, kk, vv, 0.9)
    _close(a, np.repeat(vv, 3, axis=0), 1e-15, "single key: A = v")
    _close(l, 0.9 * (q @ kk[0]), 1e-13, "single key: L = s q.k")

    m = 7
    krow = rng.standard_normal(d)
    kk = np.tile(krow, (m, 1))
    vv = rng.standard_normal((m, 3))
    a, l = attention(q, kk, vv, 0.4)
    _close(a, np.tile(vv.mean(axis=0), (3, 1)), 1e-14, "identical keys: A = mean(V)")
    _close(l, 0.4 * (q @ krow) + math.log(m), 1e-13, "identical keys: L = s q.k + log m")

    kk = rng.standard_normal((6, d))
    vconst = rng.standard_normal(3)
    a, _ = attention(q, kk, np.tile(vconst, (6, 1)), 1.1)
    _close(a, np.tile(vconst, (3, 1)), 1e-14, "constant values: A = v")

    vv = rng.standard_normal((6, 3))
    a, l = attention(np.zeros((2, d)), kk, vv, 1.0)
    _close(a, np.tile(vv.mean(axis=0), (2, 1)), 1e-14, "zero query: A = mean(V)")
    _close(l, np.full(2, math.log(6)), 1e-14, "zero query: L = log m")

    w = rng.standard_normal(d)
    a0, l0 = attention(q, kk, vv, 0.6)
    a1, l1 = attention(q, kk + w, vv, 0.6)
    _close(a1, a0, 1e-13, "shifted keys: A unchanged")
    _close(l1, l0 + 0.6 * (q @ w), 1e-13, "shifted keys: L + s q.w")

    a, l = attention(q, np.zeros((0, d)), np.zeros((0, 4)), 1.0)
    _close(a, np.zeros((3, 4)), 0.0, "empty key set: A = 0")
    assert np.all(np.isneginf(l)), "empty key set: L = -inf"

    ex = json.load(open(os.path.join(GOLDEN, "merge_worked_examples.json")))
    for case in ex["attention"]:
        a, l = attention(np.array(case["q"]), np.array(case["k"]), np.array(case["v"]), case["scale"])
        _close(a, case["a"], 1e-15, f"worked example {case['name']} A")
        _close(l, case["l"], 1e-15, f"worked example {case['name']} L")


# ----------------------------------------------------------------------------
# merge
# ----------------------------------------------------------------------------

def _val(x):
    return -np.inf if x == "-inf" else x


def check_merge(merge, attention):
    rng = np.random.default_rng(11)
    for seed in range(6):
        r = np.random.default_rng(100 + seed)
        n, m, d = 5, int(r.integers(2, 40)), 8
        q = r.standard_normal((n, d)) * 1.5
        k = r.standard_normal((m, d))
        v = r.standard_normal((m, d))
        cut = int(r.integers(1, m))
        af, lf = attention(q, k, v, 1 / math.sqrt(d))
        a1, l1 = attention(q, k[:cut], v[:cut], 1 / math.sqrt(d))
        a2, l2 = attention(q, k[cut:], v[cut:], 1 / math.sqrt(d))
        am, lm = merge(a1, l1, a2, l2)
        _close(am, af, 1e-12, f"split identity A (seed {seed}, cut {cut}/{m})")
        _close(lm, lf, 1e-12, f"split identity L (seed {seed})")
        bm, blm = merge(a2, l2, a1, l1)
        _close(bm, am, 1e-13, "commutativity A")
        _close(blm, lm, 1e-13, "commutativity L")
        if m >= 3:
            c1, c2 = sorted(r.choice(np.arange(1, m), size=2, replace=False))
            p = [attention(q, k[s:e], v[s:e], 1 / math.sqrt(d))
                 for s, e in ((0, c1), (c1, c2), (c2, m))]
            left = merge(*merge(*p[0], *p[1]), *p[2])
            right = merge(*p[0], *merge(*p[1], *p[2]))
            _close(left[0], af, 1e-12, "three-way split, left fold")
            _close(right[0], af, 1e-12, "three-way split, right fold")
            _close(left[1], lf, 1e-12, "three-way L")
            _close(right[1], lf, 1e-12, "three-way L, right fold")
        ae, le = attention(q, np.zeros((0, d)), np.zeros((0, d)), 1.0)
        an, ln = merge(a1, l1, ae, le)
        _close(an, a1, 0.0, "empty set neutral A")
        _close(ln, l1, 0.0, "empty set neutral L")
        an, ln = merge(ae, le, a1, l1)
        _close(an, a1, 0.0, "empty set neutral A (left)")
        aa, la = merge(a1, l1, a1, l1)
        _close(aa, a1, 1e-15, "self-merge A unchanged")
        _close(la, l1 + math.log(2), 1e-14, "self-merge L + log 2")
    # extreme normaliser gaps do not overflow
    a1 = rng.standard_normal((3, 4))
    a2 = rng.standard_normal((3, 4))
    am, lm = merge(a1, np.full(3, 800.0), a2, np.full(3, 0.0))
    _close(am, a1, 1e-15, "dominant side wins")
    _close(lm, np.full(3, 800.0), 1e-12, "dominant side L")

    ex = json.load(open(os.path.join(GOLDEN, "merge_worked_examples.json")))
    for case in ex["merge"]:
        a, l = merge(np.array([case["a1"]]), np.array([_val(case["l1"])]),
                     np.array([case["a2"]]), np.array([_val(case["l2"])]))
        _close(a[0], case["a"], 1e-15, f"worked example {case['name']} A")
        lv = _val(case["l"])
        if lv == -np.inf:
            assert np.isneginf(l[0]), f"worked example {case['name']} L"
        else:
            _close(l[0], lv, 1e-15, f"worked example {case['name']} L")
    for case in ex["split"]:
        ao, lo = attention(np.array(case["q"]), np.array(case["k_out"]), np.array(case["v_out"]), case["scale"])
        ai, li = attention(np.array(case["q"]), np.array(case["k_in"]), np.array(case["v_in"]), case["scale"])
        _close(ao, case["a_out"], 1e-15, "worked split A_out")
        _close(lo, case["l_out"], 1e-15, "worked split L_out")
        _close(ai, case["a_in"], 1e-15, "worked split A_in")
        _close(li, case["l_in"], 1e-15, "worked split L_in")
        af, lf = merge(ao, lo, ai, li)
        _close(af, case["a_full"], 1e-15, "worked split A_full")
        _close(lf, case["l_full"], 1e-15, "worked split L_full")


# ----------------------------------------------------------------------------
# gates
# ----------------------------------------------------------------------------

def count_by_loop(cur, prev):
    """Pure-Python element loop: positions with any differing element."""
    B, nb = cur[0].shape[0], cur[0].shape[1]
    out = []
    for b in range(B):
        cnt = 0
        for p in range(nb):
            hit = False
            for c, pr in zip(cur, prev):
                a = c[b, p].reshape(-1).tolist()
                bb = pr[b, p].reshape(-1).tolist()
                if any(x != y for x, y in zip(a, bb)):
                    hit = True
            cnt += hit
        out.append(cnt)
    return np.array(out)


def check_count_gate(update_count, gate_count, make_schedule):
    # M against the generator's own record and against an element loop
    for kw in (dict(schedule="redraw", redraw_range=(1, 4), B=2, nb=32),
               dict(schedule="unmask", unmask_range=(1, 2), B=1, nb=8),
               dict(schedule="poisson", poisson_lam=3.0, B=3, nb=16)):
        s = make_schedule(dtype="bf16", hq=4, hkv=2, d=8, lp=16, steps=12, seed=21, **kw)
        for t in range(1, s.steps + 1):
            cur = [s.q[t], s.k[t], s.v[t]]
            prev = [s.q[t - 1], s.k[t - 1], s.v[t - 1]]
            m = update_count(cur, prev)
            assert np.array_equal(m, s.touched[t]), f"M {m} vs generator {s.touched[t]} ({kw['schedule']}, t={t})"
            assert np.array_equal(m, count_by_loop(cur, prev)), "M vs element loop"
    # a change in only K, or only V, or one element of one head, counts
    base = np.zeros((1, 4, 2, 3), dtype=np.float32)
    for which in range(3):
        cur = [base.copy(), base.copy(), base.copy()]
        cur[which][0, 2, 1, 2] = 1.0
        m = update_count(cur, [base, base, base])
        assert m.tolist() == [1], f"single element change in operand {which}: M = {m}"
    # -0.0 vs +0.0 differ bitwise
    cur = [base.copy(), base, base]
    cur[0][0, 1, 0, 0] = -0.0
    assert update_count(cur, [base, base, base]).tolist() == [1], "bitwise compare of -0.0"
    # strict inequality and the invalid cache
    m = np.array([0, 3, 4, 5])
    dec = gate_count(m, 4, True, 3)
    assert dec.shape == (4, 3)
    assert dec[:, 0].tolist() == [1, 1, 0, 0], f"M < tau: {dec[:, 0]}"
    assert np.all(dec == dec[:, :1]), "count gate is per sequence"
    assert not gate_count(m, 4, False, 3).any(), "first step recomputes"
    assert gate_count(np.array([0]), 0, True, 1).tolist() == [[0]], "tau = 0 never reuses"


def check_cosine_gate(head_cosine, gate_cosine):
    # exact tie: cos((3,4),(4,3)) = 24/25, the double nearest 0.96
    q = np.zeros((1, 1, 1, 2))
    p = np.zeros((1, 1, 1, 2))
    q[0, 0, 0] = [3.0, 4.0]
    p[0, 0, 0] = [4.0, 3.0]
    cos, zero = head_cosine(q, p)
    assert cos[0, 0] == 0.96, f"cos {cos[0, 0]!r} != 0.96"
    assert gate_cosine(cos, zero, 0.96, True).tolist() == [[0]], "tie recomputes"
    assert gate_cosine(cos, zero, 0.9599, True).tolist() == [[1]], "above gamma reuses"
    assert gate_cosine(cos, zero, 0.9599, False).tolist() == [[0]], "invalid cache recomputes"
    # identical -> 1; orthogonal -> 0; opposite -> -1
    r = np.random.default_rng(5)
    x = r.standard_normal((2, 6, 3, 4))
    cos, zero = head_cosine(x, x.copy())
    _close(cos, np.ones((2, 3)), 1e-15, "identical Q: cos = 1")
    cos, _ = head_cosine(x, -x)
    _close(cos, -np.ones((2, 3)), 1e-15, "opposite Q: cos = -1")
    # zero norm -> recompute even with gamma below any cosine
    z = x.copy()
    z[1, :, 2, :] = 0.0
    cos, zero = head_cosine(z, x)
    assert zero[1, 2] and not zero[0, 0]
    dec = gate_cosine(cos, zero, -2.0, True)
    assert dec[1, 2] == 0 and dec[0, 0] == 1, "zero norm recomputes"
    # per-head, per-sequence independence: against mpmath over each head's values
    y = x + 0.3 * r.standard_normal(x.shape)
    cos, _ = head_cosine(y, x)
    with mpmath.workdps(40):
        for b in range(2):
            for h in range(3):
                a = [mpmath.mpf(v) for v in y[b, :, h, :].ravel()]
                c = [mpmath.mpf(v) for v in x[b, :, h, :].ravel()]
                ref = mpmath.fsum(u * w for u, w in zip(a, c)) / (
                    mpmath.sqrt(mpmath.fsum(u * u for u in a)) * mpmath.sqrt(mpmath.fsum(w * w for w in c)))
                assert abs(cos[b, h] - float(ref)) <= 4e-16, f"cos[{b},{h}] vs mpmath"


# ----------------------------------------------------------------------------
# packing
# ----------------------------------------------------------------------------

def check_pack(varlen_pack):
    rng = np.random.default_rng(3)
    cases = [(np.array([4, 8, 16, 32, 64, 128]), None),
             (np.array([3, 0, 5, 1]), None),
             (np.array([5, 7]), np.ones(12, dtype=np.uint8)),
             (np.array([5, 7]), np.zeros(12, dtype=np.uint8))]
    for bs, locked in cases:
        n = int(bs.sum())
        if locked is None:
            locked = (rng.random(n) < 0.3).astype(np.uint8)
        cu, gather, total = varlen_pack(locked, bs)
        starts = np.concatenate([[0], np.cumsum(bs)])
        counts = np.array([int((locked[starts[b]:starts[b + 1]] == 0).sum()) for b in range(bs.size)])
        assert cu.tolist() == [0] + np.cumsum(counts).tolist(), "cu_seqlens = exclusive prefix sum of u_b"
        assert total == int((locked == 0).sum()) == len(gather), "total = number of unlocked positions"
        for b in range(bs.size):
            seg = gather[cu[b]:cu[b + 1]]
            assert np.all((seg >= starts[b]) & (seg < starts[b + 1])), "row stays in its branch"
            assert np.all(np.diff(seg) > 0), "ascending within a branch"
        assert np.all(locked[gather] == 0), "only unlocked positions are packed"
        assert sorted(gather.tolist()) == np.flatnonzero(locked == 0).tolist(), "every unlocked position once"
        x = rng.standard_normal((n, 3))
        back = np.zeros_like(x)
        back[gather] = x[gather]
        assert np.array_equal(back[locked == 0], x[locked == 0]), "gather/scatter round trip"


def check_cumulative_gate(cumulative_gates):
    """Count gate since the last refresh: a hand-worked schedule and
    invariants against the per-step count and a sticky per-position mark."""
    # One sequence of 4 positions, tau = 3; positions updated into steps
    # 1..7: {2}, {0}, {1}, {1}, {2, 3}, {}, {3}.  Step 1 has no cache
    # (recompute; the count starts again after it); steps 2-4 count {0},
    # {0,1}, {0,1}: reuse; step 5 counts {0,1,2,3} = 4 >= 3: recompute; step 6
    # counts nothing, step 7 {3}.  The per-step count (1, 1, 1, 1, 2, 0, 1)
    # would have reused at every step after the first.
    sets = [None, {2}, {0}, {1}, {1}, {2, 3}, set(), {3}]
    changed = [None] + [np.array([[p in s_ for p in range(4)]]) for s_ in sets[1:]]
    g = cumulative_gates(changed, tau=3, hq=2)
    assert [int(x["m"][0]) for x in g[1:]] == [1, 1, 2, 2, 4, 0, 1]
    assert [int(x["decision"][0, 0]) for x in g[1:]] == [0, 1, 1, 1, 0, 1, 1]
    assert all((x["decision"][:, 0:1] == x["decision"]).all() for x in g[1:])
    # Random update sets: never below the per-step count, equal to it right
    # after a refresh; tau = 0 (always recompute) makes the two identical;
    # with tau above Nb it is the union of every update since step 1; and it
    # equals a sticky per-position mark cleared on each recompute.
    r = np.random.default_rng(4)
    B, nb, S = 3, 10, 12
    changed = [None] + [r.random((B, nb)) < 0.15 for _ in range(S)]
    for tau in (0, 2, 4, nb + 1):
        g = cumulative_gates(changed, tau=tau, hq=1)
        mark = np.zeros((B, nb), dtype=bool)
        for t in range(1, S + 1):
            step = changed[t].sum(axis=1)
            m = g[t]["m"]
            assert (m >= step).all()
            if t == 1 or tau == 0:
                assert (m == step).all()
            else:
                prev_re = g[t - 1]["decision"][:, 0] == 0
                assert (m[prev_re] == step[prev_re]).all()
            if tau == nb + 1 and t > 1:
                union = np.zeros((B, nb), dtype=bool)
                for s_ in range(2, t + 1):
                    union |= changed[s_]
                assert (m == union.sum(axis=1)).all()
            mark |= changed[t]
            assert (m == mark.sum(axis=1)).all()
            assert (g[t]["decision"][:, 0] == ((m < tau) & (t > 1))).all()
            mark[g[t]["decision"][:, 0] == 0] = False


def check_rows_changed(rows_changed):
    """The rows a partial refresh recomputes: a Q change in any head marks
    its position, K/V changes do not count, nothing else is marked."""
    r = np.random.default_rng(6)
    q0 = r.integers(0, 1 << 16, size=(2, 6, 4, 8), dtype=np.uint16)
    assert not rows_changed(q0.copy(), q0).any()
    q = q0.copy()
    q[1, 4, 3, 7] ^= 1
    q[0, 0, 0, 0] ^= 0x8000
    got = rows_changed(q, q0)
    assert got.shape == (2, 6) and got.sum() == 2 and got[1, 4] and got[0, 0]
    f = r.standard_normal((1, 3, 2, 4)).astype(np.float32)
    g = f.copy()
    g[0, 2, 1, 3] = np.nextafter(g[0, 2, 1, 3], np.float32(np.inf))
    assert rows_changed(g, f).tolist() == [[False, False, True]]
