"""CPU tests: the oracle against its pins (no GPU, no library)."""

import math

import numpy as np
import pytest

import oracle
from workloads import make_block_schedule, make_varlen_batch, round_to_bf16_bits, bf16_bits_to_f32
from tests import oracle_pins as pins


def test_attention_pins():
    pins.check_attention(oracle.attention)


def test_merge_pins():
    pins.check_merge(oracle.merge, oracle.attention)


def test_count_gate_pins():
    pins.check_count_gate(oracle.update_count, oracle.gate_count, make_block_schedule)


def test_cosine_gate_pins():
    pins.check_cosine_gate(oracle.head_cosine, oracle.gate_cosine)


def test_pack_pins():
    pins.check_pack(oracle.varlen_pack)


def test_merge_many_is_n_way_split():
    r = np.random.default_rng(9)
    q = r.standard_normal((4, 16))
    k = r.standard_normal((100, 16))
    v = r.standard_normal((100, 16))
    cuts = [0, 7, 30, 31, 64, 100]
    parts = [oracle.attention(q, k[a:b], v[a:b], 0.25) for a, b in zip(cuts[:-1], cuts[1:])]
    am, lm = oracle.merge_many(parts)
    af, lf = oracle.attention(q, k, v, 0.25)
    np.testing.assert_allclose(am, af, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lm, lf, atol=1e-12, rtol=0)


# ----------------------------------------------------------------------------
# the block schedule as a whole
# ----------------------------------------------------------------------------

def _small(schedule="redraw", gate="count", **kw):
    base = dict(dtype="bf16", B=2, hq=4, hkv=2, d=16, lp=40, nb=12, steps=6, std=1.0,
                schedule=schedule, gate=gate, tau=3, gamma=0.95, seed=31)
    base.update(kw)
    return make_block_schedule(**base)


@pytest.mark.parametrize("schedule,gate", [("redraw", "count"), ("poisson", "count"),
                                           ("qnoise", "cosine")])
def test_run_block_fresh_cache_is_exact(schedule, gate):
    """Where a (b, h) recomputes, A_full is attention over prefix + block."""
    s = _small(schedule=schedule, gate=gate, redraw_range=(0, 5), poisson_lam=2.5,
               sigma_range=(0.01, 0.6))
    out = oracle.run_block(s, exact=True)
    B, nb = s.B, s.nb
    for t in range(1, s.steps + 1):
        dec = out[t]["gate"]["decision"]
        if t == 1:
            assert not dec.any(), "first step recomputes"
        af = out[t]["a_full"].reshape(B, nb, s.hq, s.d)
        ae = out[t]["a_exact"].reshape(B, nb, s.hq, s.d)
        for b in range(B):
            for h in range(s.hq):
                if dec[b, h] == 0:
                    np.testing.assert_allclose(af[b, :, h], ae[b, :, h], atol=1e-12, rtol=0)


def test_run_block_reuse_staleness_invariant():
    """On a reuse step, rows whose Q is unchanged since the last refresh get
    the exact result; at least one updated row does not (reuse happened)."""
    s = _small(schedule="redraw", redraw_range=(1, 2), tau=3, steps=6)
    out = oracle.run_block(s, exact=True)
    gates = [None] + [out[t]["gate"] for t in range(1, s.steps + 1)]
    last = oracle.refresh_steps(gates, s.steps)
    saw_reuse = saw_stale = False
    for t in range(2, s.steps + 1):
        dec = out[t]["gate"]["decision"]
        af = out[t]["a_full"].reshape(s.B, s.nb, s.hq, s.d)
        ae = out[t]["a_exact"].reshape(s.B, s.nb, s.hq, s.d)
        for b in range(s.B):
            for h in range(s.hq):
                if dec[b, h] != 1:
                    continue
                saw_reuse = True
                tr = last[t][b, h]
                same = np.all(s.q[t][b, :, h] == s.q[tr][b, :, h], axis=-1)
                np.testing.assert_allclose(af[b, same, h], ae[b, same, h], atol=1e-12, rtol=0)
                if (~same).any():
                    diff = np.abs(af[b, ~same, h] - ae[b, ~same, h]).max()
                    saw_stale |= diff > 1e-6
    assert saw_reuse and saw_stale


def test_run_block_gqa_equals_repeated_heads():
    """Query head h reads KV head h // G: the GQA result equals MHA with the
    KV heads repeated G times (the standard grouped-query definition)."""
    s = _small(schedule="redraw", hq=6, hkv=2, B=1, steps=3)
    g = s.hq // s.hkv
    m = _small(schedule="redraw", hq=6, hkv=6, B=1, steps=3)
    m.kp = np.repeat(s.kp, g, axis=1)
    m.vp = np.repeat(s.vp, g, axis=1)
    m.q = s.q
    m.k = [np.repeat(x, g, axis=2) for x in s.k]
    m.v = [np.repeat(x, g, axis=2) for x in s.v]
    a = oracle.run_block(s)
    b = oracle.run_block(m)
    for t in range(1, 4):
        np.testing.assert_array_equal(a[t]["a_full"], b[t]["a_full"])
        np.testing.assert_array_equal(a[t]["l_full"], b[t]["l_full"])


def test_run_block_tau_decisions_follow_counts():
    s = make_block_schedule(dtype="f32", B=1, hq=4, hkv=4, d=64, lp=256, nb=32, steps=8,
                            schedule="redraw", redraw_range=(1, 4), gate="count", tau=4, seed=1)
    g = oracle.step_gates(s)
    for t in range(1, 9):
        m = g[t]["m"][0]
        assert m == s.touched[t, 0]
        want = 0 if t == 1 else int(m < 4)
        assert np.all(g[t]["decision"] == want)


def test_run_varlen_matches_full_attention_with_locked_keys():
    vb = make_varlen_batch(block_sizes=(3, 0, 5, 8), prefix_lens=(7, 4, 0, 9), h=2, d=8,
                           lock_p=0.4, seed=12, std=1.0)
    res = oracle.run_varlen(vb)
    bstart = np.concatenate([[0], np.cumsum(vb.block_sizes)])
    pstart = np.concatenate([[0], np.cumsum(vb.prefix_lens)])
    f = lambda x: bf16_bits_to_f32(x).astype(np.float64)  # noqa: E731
    for b in range(vb.block_sizes.size):
        for r in range(res["cu_seqlens"][b], res["cu_seqlens"][b + 1]):
            p = res["gather_idx"][r]
            for h in range(vb.h):
                k = np.concatenate([f(vb.kp[h, pstart[b]:pstart[b + 1]]), f(vb.k[bstart[b]:bstart[b + 1], h])])
                v = np.concatenate([f(vb.vp[h, pstart[b]:pstart[b + 1]]), f(vb.v[bstart[b]:bstart[b + 1], h])])
                a, l = oracle.attention(f(vb.q[p, h])[None], k, v, vb.scale)
                np.testing.assert_allclose(res["a_full"][r, h], a[0], atol=1e-12, rtol=0)
                np.testing.assert_allclose(res["l_full"][r, h], l[0], atol=1e-12, rtol=0)
    # branch 2 has an empty prefix: L_out = -inf and A_full = A_in
    r0, r1 = res["cu_seqlens"][2], res["cu_seqlens"][3]
    assert r1 > r0
    assert np.all(np.isneginf(res["l_out"][r0:r1]))
    np.testing.assert_array_equal(res["a_full"][r0:r1], res["a_in"][r0:r1])


# ----------------------------------------------------------------------------
# the generator (input plumbing only)
# ----------------------------------------------------------------------------

def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    r = np.random.default_rng(2)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32) * 3,
                        np.array([1.00390625, 1.01171875, -2.00390625, 0.0, -0.0], dtype=np.float32)])
    ours = round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generator_is_seeded_and_shaped():
    a = _small(seed=5)
    b = _small(seed=5)
    c = _small(seed=6)
    assert np.array_equal(a.kp, b.kp) and np.array_equal(a.q[-1], b.q[-1])
    assert not np.array_equal(a.kp, c.kp)
    assert a.kp.shape == (2, 2, 40, 16) and a.q[0].shape == (2, 12, 4, 16)
    assert a.k[3].shape == (2, 12, 2, 16) and a.kp.dtype == np.uint16
    assert math.isclose(a.scale, 0.25)


def test_key_blocks_cover_the_prefix_once():
    # a selected list and its complement cover every prefix key exactly once,
    # the last (ragged) block clipped to the prefix length
    from workloads import make_key_block_lists
    lp = 64 * 9 + 17
    sel, rest = make_key_block_lists(B=2, hkv=3, lp=lp, density=0.4, seed=5)
    assert sel.shape == (2, 3, 4) and rest.shape == (2, 3, 6)
    for b in range(2):
        for g in range(3):
            keys = np.concatenate([oracle.block_keys(sel[b, g], lp), oracle.block_keys(rest[b, g], lp)])
            assert np.array_equal(np.sort(keys), np.arange(lp))
    assert oracle.block_keys([9], lp).tolist() == list(range(576, lp))
    assert oracle.block_keys([], lp).size == 0


def test_sparse_residual_split_is_exact():
    # [FB] sparse attention with the unselected keys as the cached "out" set:
    # merging the selected-block pass with the complementary (residual) pass
    # is attention over the whole prefix (to rounding); an empty selection
    # weighs nothing
    from workloads import make_key_block_lists
    s = make_block_schedule(dtype="bf16", B=1, hq=4, hkv=2, d=32, lp=64 * 7 + 5, nb=6, steps=0, std=1.0,
                            schedule="none", seed=12)
    sel, rest = make_key_block_lists(B=1, hkv=2, lp=s.lp, density=0.3, seed=2)
    for h in range(4):
        a1, l1 = oracle.prefix_rows_in_blocks(s, 0, 0, h, sel[0, h // 2])
        a2, l2 = oracle.prefix_rows_in_blocks(s, 0, 0, h, rest[0, h // 2])
        am, lm = oracle.merge(a1, l1, a2, l2)
        af, lf = oracle.prefix_rows(s, 0, 0, h)
        assert np.max(np.abs(am - af)) < 1e-12 and np.max(np.abs(lm - lf)) < 1e-12
        a0, l0 = oracle.prefix_rows_in_blocks(s, 0, 0, h, [])
        assert np.all(a0 == 0) and np.all(np.isneginf(l0))
        ae, le = oracle.merge(a0, l0, af, lf)
        assert np.max(np.abs(ae - af)) < 1e-15 and np.max(np.abs(le - lf)) < 1e-15


def test_kl_pins():
    # [SL] the lock criterion: KL(p || q) of the two steps' posteriors.
    # Closed forms: identical rows (and a constant shift of a row) give 0;
    # p = (1/2, 1/2) against q = (1/4, 3/4) gives ln(4/3) / 2; a uniform p
    # over V against q putting e^c on one entry gives the closed form below;
    # a zero-probability entry of p adds nothing; q = 0 where p > 0 is +inf.
    x = np.array([[0.3, -1.2, 2.0, 0.0]])
    assert abs(oracle.kl_rows(x, x)[0]) < 1e-15
    assert abs(oracle.kl_rows(x, x + 5.0)[0]) < 1e-14
    got = oracle.kl_rows(np.array([[0.0, 0.0]]), np.array([[0.0, math.log(3.0)]]))[0]
    assert abs(got - 0.5 * math.log(4.0 / 3.0)) < 1e-15
    V, c = 7, 1.7
    y = np.zeros((1, V)); y[0, 2] = c
    want = -math.log(V) + math.log(V - 1 + math.exp(c)) - c / V
    assert abs(oracle.kl_rows(np.zeros((1, V)), y)[0] - want) < 1e-14
    assert abs(oracle.kl_rows(np.array([[0.0, -np.inf]]), np.array([[0.0, 0.0]]))[0] - math.log(2.0)) < 1e-15
    assert oracle.kl_rows(np.array([[0.0, 0.0]]), np.array([[0.0, -np.inf]]))[0] == np.inf
    # Gibbs: KL >= 0, and it grows with the drift of the previous row
    r = np.random.default_rng(1)
    a = r.standard_normal((1, 50)) * 3
    kls = [oracle.kl_rows(a, a + s * r.standard_normal((1, 50)))[0] for s in (0.01, 0.1, 1.0)]
    assert 0 <= kls[0] < kls[1] < kls[2]
    # a lock is sticky, and only eligible tokens lock
    upd = oracle.lock_update([1, 0, 0, 0], [0, 1, 0, 1], np.array([9.0, 0.1, 0.0, 2.0]), 0.5)
    assert upd.tolist() == [1, 1, 0, 0]


def test_cumulative_gate_pins():
    pins.check_cumulative_gate(oracle.cumulative_gates)


def test_rows_changed_pins():
    pins.check_rows_changed(oracle.rows_changed)


def test_partial_refresh_is_exact():
    # A_out/L_out of a row depend on its query only, so refreshing just the
    # rows whose Q changed keeps the whole cache equal to a full recompute
    # with the current Q at every step (to rounding of the row subset).
    s = make_block_schedule(B=2, hq=4, hkv=2, d=16, lp=37, nb=6, steps=5, schedule="redraw",
                            redraw_range=(1, 2), seed=12)
    steps = oracle.run_block(s, partial=True)
    for t in range(1, s.steps + 1):
        for b in range(s.B):
            for h in range(s.hq):
                a, l_ = oracle.prefix_rows(s, t, b, h)
                np.testing.assert_allclose(steps[t]["a_out"].reshape(s.B, s.nb, s.hq, s.d)[b, :, h], a,
                                           rtol=0, atol=1e-12)
                np.testing.assert_allclose(steps[t]["l_out"].reshape(s.B, s.nb, s.hq)[b, :, h], l_,
                                           rtol=0, atol=1e-12)
    # with no Q change after step 1 nothing is recomputed
    n = make_block_schedule(B=1, hq=2, hkv=2, d=16, lp=20, nb=4, steps=3, schedule="none", seed=3)
    st = oracle.run_block(n, partial=True)
    assert np.array_equal(st[1]["a_out"], st[3]["a_out"])
