"""GPU parity at the full sizes of the five workloads, in the launch
configuration the benchmark uses (whole block schedules through the step
driver, replayed from a captured HIP graph where the benchmark does so).

Gate decisions and update counts are compared bit-exactly at every step.
Outputs are compared with the CPU oracle on all rows where the oracle is
cheap (the LLaDA-like and float32 workloads) and on sampled rows computed one
by one elsewhere; a sampled row's cached prefix part is recomputed by the
oracle from the Q of the step that last refreshed its head.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import preset
from tests.gpu_util import DEV, check_a, check_l, dev_bits, dev_in, host

pytestmark = pytest.mark.gpu

ba = pytest.importorskip("cached_split_attention_amd")


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _to_dev(sched):
    return ([dev_in(x, sched.dtype) for x in sched.q], [dev_in(x, sched.dtype) for x in sched.k],
            [dev_in(x, sched.dtype) for x in sched.v])


def _sampled_rows(sched, t, gates_hist, last, rows, got_a, got_l):
    """Oracle A_full/L_full of the sampled (b, h, i) rows at step t."""
    for b, h, i in rows:
        tr = int(last[t][b, h])
        ao, lo = oracle.prefix_rows(sched, tr, b, h, rows=[i])
        ai, li = oracle.block_rows(sched, t, b, h, rows=[i])
        af, lf = oracle.merge(ao, lo, ai, li)
        r = b * sched.nb + i
        check_a(got_a[r, h][None], af, f"A_full step {t} (b{b} h{h} i{i})")
        check_l(got_l[r, h][None], lf, f"L_full step {t} (b{b} h{h} i{i})")


def _check_whole_heads(sched, t, pairs, last, attn, cache, name):
    """Every row of the (b, h) pairs at step t against the oracle: A_in/L_in
    over the block, the cached A_out/L_out (prefix part with the Q of the step
    that last refreshed the head), and their merge A_full/L_full."""
    nb, hq, d = sched.nb, sched.hq, sched.d
    ga_in, gl_in = host(attn.a_in).reshape(-1, hq, d), host(attn.l_in).reshape(-1, hq)
    ga_out, gl_out = host(attn.a_out).reshape(-1, hq, d), host(attn.l_out).reshape(-1, hq)
    ga_f, gl_f = host(attn.a_full).reshape(-1, hq, d), host(attn.l_full).reshape(-1, hq)
    for b, h in pairs:
        tr = int(last[t][b, h])
        key = (tr, b, h)
        if key not in cache:
            cache[key] = oracle.prefix_rows(sched, tr, b, h)
        ao, lo = cache[key]
        ai, li = oracle.block_rows(sched, t, b, h)
        af, lf = oracle.merge(ao, lo, ai, li)
        rs = slice(b * nb, (b + 1) * nb)
        what = f"[{name}] step {t} b{b} h{h} (refreshed at step {tr}), all {nb} rows"
        check_a(ga_in[rs, h], ai, "A_in " + what)
        check_l(gl_in[rs, h], li, "L_in " + what)
        check_a(ga_out[rs, h], ao, "A_out " + what)
        check_l(gl_out[rs, h], lo, "L_out " + what)
        check_a(ga_f[rs, h], af, "A_full " + what)
        check_l(gl_f[rs, h], lf, "L_full " + what)
    say(f"[{name}] step {t}: every row of {len(pairs)} (sequence, head) pairs checked")


def _run_schedule_checked(name, rows_per_step=8, full_rows=False, use_graph=False, seed=0, whole=None,
                          use_mask=False, **overrides):
    """whole(sched, gates) -> {step: [(b, h), ...]}: (sequence, head) pairs
    whose every row is checked at that step, besides the sampled rows.
    use_mask: the count gate is fed the generator's record of rewritten
    positions (a caller's update mask) instead of comparing rows; decisions
    and M must still equal the oracle's row comparison."""
    sched = preset(name, **overrides)
    say(f"[{name}] B={sched.B} Hq={sched.hq} Hkv={sched.hkv} d={sched.d} Lp={sched.lp} Nb={sched.nb} "
        f"steps={sched.steps} gate={sched.gate}")
    gates = oracle.step_gates(sched)
    last = oracle.refresh_steps(gates, sched.steps)
    if sched.gate == "cosine":
        margins = [np.abs(gates[t]["cos"] - sched.gamma).min() for t in range(2, sched.steps + 1)]
        assert min(margins) > 1e-6, f"seed gives a near-tie cosine ({min(margins):.2e})"
    q, k, v = _to_dev(sched)
    masks = ([None] + [torch.from_numpy(sched.rewritten[t]).to(DEV) for t in range(1, sched.steps + 1)]
             if use_mask else None)
    kp, vp = dev_in(sched.kp, sched.dtype), dev_in(sched.vp, sched.dtype)
    attn = ba.CachedBlockAttention(kp, vp, nb=sched.nb, hq=sched.hq, gate=sched.gate, tau=sched.tau,
                                   gamma=sched.gamma, scale=sched.scale)
    ref_full = oracle.run_block(sched) if full_rows else None
    whole_at = whole(sched, gates) if whole is not None else {}
    prefix_cache = {}
    rng = np.random.default_rng(seed)
    outs = []
    if use_graph:
        # step-by-step graphs, as replayed by the benchmark's per-step legs,
        # and the whole-block graph it times
        g = attn.capture_block(q, k, v, masks=masks)
        g.replay()
        torch.cuda.synchronize()
        say(f"[{name}] whole-block graph replayed")
        final = (host(attn.a_full), host(attn.l_full), attn.decision.cpu().numpy())
        attn.start_block()
    recomputes = 0
    for t in range(1, sched.steps + 1):
        af, lf = attn.step(q[t], k[t], v[t], q[t - 1], k[t - 1], v[t - 1],
                           upd_mask=None if masks is None else masks[t])
        torch.cuda.synchronize()
        dec = attn.decision.cpu().numpy()
        assert np.array_equal(dec, gates[t]["decision"]), f"[{name}] step {t}: decisions differ"
        if sched.gate in ("count", "count_cum"):
            assert np.array_equal(attn.m_count.cpu().numpy(), gates[t]["m"]), f"[{name}] step {t}: M differs"
        assert attn.waits_given_up() == 0, f"[{name}] step {t}: a prefix workgroup gave up waiting for its gate"
        recomputes += int((dec == 0).sum())
        if t in whole_at:
            _check_whole_heads(sched, t, whole_at[t], last, attn, prefix_cache, name)
        ga, gl = host(af), host(lf)
        if full_rows:
            check_a(ga, ref_full[t]["a_full"], f"[{name}] A_full step {t}")
            check_l(gl, ref_full[t]["l_full"], f"[{name}] L_full step {t}")
        else:
            rows = [(int(rng.integers(sched.B)), int(rng.integers(sched.hq)), int(rng.integers(sched.nb)))
                    for _ in range(rows_per_step)]
            # always include the last row (ragged tail of the block tile)
            rows.append((sched.B - 1, sched.hq - 1, sched.nb - 1))
            _sampled_rows(sched, t, gates, last, rows, ga.reshape(-1, sched.hq, sched.d),
                          gl.reshape(-1, sched.hq))
        outs.append((ga, gl))
    say(f"[{name}] {sched.steps} steps checked, {recomputes} (b, h) prefix recomputes")
    if use_graph:
        assert np.array_equal(final[2], dec)
        np.testing.assert_array_equal(final[0], outs[-1][0])
        np.testing.assert_array_equal(final[1], outs[-1][1])
    return sched, recomputes


def test_workload_tiny_f32():
    _run_schedule_checked("c1_tiny_f32", full_rows=True, use_graph=True)


def test_workload_llada():
    _run_schedule_checked("c2_llada", full_rows=True, use_graph=True)


def _gqa_whole(sched, gates):
    # A sequence with a gated recompute: every head and row of it at the
    # first step, at its gated recompute, at the next step (which reuses it)
    # and at the last step; plus one (sequence, KV head) group of another
    # sequence (its 4 query heads) at the gated recompute step.
    rec = [(t, b) for t in range(2, sched.steps + 1) for b in range(sched.B)
           if (gates[t]["decision"][b] == 0).all()]
    assert rec, "the schedule has no gated recompute"
    t_r, b = rec[0]
    t_u = next(t for t in range(t_r + 1, sched.steps + 1) if gates[t]["decision"][b].all())
    g = sched.hq // sched.hkv
    b2 = (b + 1) % sched.B
    heads = [(b, h) for h in range(sched.hq)]
    out = {1: heads, t_r: heads + [(b2, h) for h in range(2 * g, 3 * g)], t_u: heads, sched.steps: heads}
    return out


def test_workload_gqa_long_context():
    sched, rec = _run_schedule_checked("c3_gqa_long", rows_per_step=6, use_graph=False, seed=3, whole=_gqa_whole)
    assert rec > sched.B * sched.hq  # gated recomputes beyond the first step


def test_workload_gqa_update_mask():
    # the same schedule with the count gate reading the caller's update mask
    # (the fused launch's mask path), whole-block graph included
    sched, rec = _run_schedule_checked("c3_gqa_long", rows_per_step=4, use_graph=True, seed=5, use_mask=True)
    assert rec > sched.B * sched.hq


def _video_whole(sched, gates):
    # Every row (all 13 row tiles of the 1560-row block, its 24-row tail) of
    # two heads: one the similarity gate reuses and one it recomputes at the
    # first step that has both, checked there and at the last step.
    t1 = next(t for t in range(2, sched.steps + 1)
              if gates[t]["decision"][0].any() and not gates[t]["decision"][0].all())
    dec = gates[t1]["decision"][0]
    h_reuse, h_rec = int(np.flatnonzero(dec == 1)[0]), int(np.flatnonzero(dec == 0)[-1])
    pairs = [(0, h_reuse), (0, h_rec)]
    return {t1: pairs, sched.steps: pairs}


def test_workload_video():
    sched, rec = _run_schedule_checked("c4_video", rows_per_step=6, use_graph=False, seed=4, whole=_video_whole)
    assert sched.B * sched.hq < rec < sched.steps * sched.B * sched.hq  # some heads reuse


def test_workload_long_prefix():
    # The pages' long-context axis: the LLaDA-like heads over a 256k-token
    # prefix, four steps (many key splits per head, and their combine).
    sched, rec = _run_schedule_checked("c2_llada", rows_per_step=3, seed=6, lp=262144, steps=4)
    assert rec >= sched.B * sched.hq


def test_workload_gqa_long_prefix():
    # The long-context axis at the GQA shape: one sequence's 32 query heads
    # on 8 KV heads over a 512k-token prefix (the 256-row kernel with many
    # key splits per (sequence, KV head), and their combine), three steps.
    sched, rec = _run_schedule_checked("c3_gqa_long", rows_per_step=3, seed=9, lp=524288, B=1, steps=3)
    assert rec >= sched.B * sched.hq


def test_workload_gqa_cumulative_gate():
    # The GQA long-context schedule (Poisson(3) rewritten rows per step, tau
    # 8) gated on the positions updated since the last refresh: the
    # per-step count rarely reaches tau, the cumulative one every few steps.
    sched, rec = _run_schedule_checked("c3_gqa_long", rows_per_step=4, seed=7, gate="count_cum", steps=16)
    per_step = oracle.step_gates(preset("c3_gqa_long", steps=16))
    rec_step = sum(int((per_step[t]["decision"] == 0).sum()) for t in range(1, 17))
    assert rec > rec_step, (rec, rec_step)


def test_workload_llada_cosine_gate():
    # The per-head similarity gate on the LLaDA-like unmasking schedule (the
    # dLLM setting rather than video): decisions per (sequence, head).
    sched, rec = _run_schedule_checked("c2_llada", full_rows=True, gate="cosine", gamma=0.95, steps=16)
    assert sched.B * sched.hq < rec < sched.steps * sched.B * sched.hq


def test_workload_gqa_partial_refresh():
    # Partial refresh on the GQA long-context schedule: only rows whose Q
    # changed are recomputed, so every step's A_full equals attention over
    # prefix + block with the current Q (checked on sampled rows), and the
    # per-row marks equal the oracle's changed rows.
    sched = preset("c3_gqa_long", steps=8)
    say(f"[c3 partial] B={sched.B} Hq={sched.hq} Hkv={sched.hkv} Lp={sched.lp} Nb={sched.nb} steps={sched.steps}")
    q, k, v = _to_dev(sched)
    kp, vp = dev_in(sched.kp, sched.dtype), dev_in(sched.vp, sched.dtype)
    attn = ba.CachedBlockAttention(kp, vp, nb=sched.nb, hq=sched.hq, gate="partial", scale=sched.scale)
    rng = np.random.default_rng(8)
    g = sched.hq // sched.hkv
    redone = 0
    for t in range(1, sched.steps + 1):
        af, lf = attn.step(q[t], k[t], v[t], q[t - 1], k[t - 1], v[t - 1])
        torch.cuda.synchronize()
        ch = oracle.rows_changed(sched.q[t], sched.q[t - 1])
        want_keep = ((~ch) & (t > 1)).astype(np.uint8)
        assert np.array_equal(attn.decision.cpu().numpy(), want_keep), f"step {t}: row marks differ"
        redone += int((want_keep == 0).sum())
        ga = host(af).reshape(-1, sched.hq, sched.d)
        gl = host(lf).reshape(-1, sched.hq)
        picks = [(int(rng.integers(sched.B)), int(rng.integers(sched.hq)), int(rng.integers(sched.nb)))
                 for _ in range(5)]
        # a changed row when there is one
        bs, ps = np.nonzero(ch)
        if t > 1 and bs.size:
            picks.append((int(bs[0]), int(rng.integers(sched.hq)), int(ps[0])))
        for b, h, i in picks:
            qq = oracle.to_f64(sched.q[t][b, i:i + 1, h, :], sched.dtype)
            kk = np.concatenate([oracle.to_f64(sched.kp[b, h // g], sched.dtype),
                                 oracle.to_f64(sched.k[t][b, :, h // g], sched.dtype)])
            vv = np.concatenate([oracle.to_f64(sched.vp[b, h // g], sched.dtype),
                                 oracle.to_f64(sched.v[t][b, :, h // g], sched.dtype)])
            wa, wl = oracle.attention(qq, kk, vv, sched.scale)
            r = b * sched.nb + i
            check_a(ga[r, h][None], wa, f"A_full step {t} (b{b} h{h} i{i})")
            check_l(gl[r, h][None], wl, f"L_full step {t} (b{b} h{h} i{i})")
    say(f"[c3 partial] {sched.steps} steps checked, {redone} rows recomputed of {sched.steps * sched.B * sched.nb}")
    assert sched.B * sched.nb < redone < sched.steps * sched.B * sched.nb


def test_workload_varlen_branches():
    vb = preset("c5_varlen")
    say(f"[c5_varlen] block sizes {vb.block_sizes.tolist()} prefixes {vb.prefix_lens.tolist()} "
        f"H={vb.h} d={vb.d} locked={int(vb.locked.sum())}")
    heads = list(range(vb.h))
    ref = oracle.run_varlen(vb, heads=heads)
    dev = "cuda"
    n = int(vb.block_sizes.sum())
    nbr = vb.block_sizes.size
    cu_q = torch.empty(nbr + 1, device=dev, dtype=torch.int32)
    gather = torch.empty(n, device=dev, dtype=torch.int32)
    total = torch.empty(1, device=dev, dtype=torch.int32)
    qp = torch.zeros(n, vb.h, vb.d, device=dev, dtype=torch.bfloat16)
    ba.ba_varlen_pack(vb.block_sizes, torch.from_numpy(vb.locked).to(dev), cu_q, gather, total,
                      dev_bits(vb.q), qp)
    cu_kp = torch.from_numpy(np.concatenate([[0], np.cumsum(vb.prefix_lens)]).astype(np.int32)).to(dev)
    cu_kb = torch.from_numpy(np.concatenate([[0], np.cumsum(vb.block_sizes)]).astype(np.int32)).to(dev)
    kp, vp = dev_bits(vb.kp), dev_bits(vb.vp)
    kb, vbk = dev_bits(vb.k), dev_bits(vb.v)
    max_q = int(vb.block_sizes.max())
    a_out = torch.empty(n, vb.h, vb.d, device=dev)
    l_out = torch.empty(n, vb.h, device=dev)
    kw = dict(q_layout="thd", cu_q=cu_q, max_q=max_q)
    ws = torch.zeros(max(1, ba.ba_prefix_attn_workspace(qp, kp, vp, kv_layout="htd", cu_k=cu_kp,
                                                         max_k=int(vb.prefix_lens.max()), **kw)),
                     device=dev, dtype=torch.uint8)
    ba.ba_prefix_attn(qp, kp, vp, a_out, l_out, ws, kv_layout="htd", cu_k=cu_kp,
                      max_k=int(vb.prefix_lens.max()), **kw)
    a_full = torch.empty(n, vb.h, vb.d, device=dev)
    l_full = torch.empty(n, vb.h, device=dev)
    ba.ba_block_attn(qp, kb, vbk, a_cache=a_out, l_cache=l_out, a_full=a_full, l_full=l_full,
                     kv_layout="thd", cu_k=cu_kb, max_k=int(vb.block_sizes.max()), **kw)
    torch.cuda.synchronize()
    tot = ref["total"]
    assert int(total.item()) == tot
    assert cu_q.cpu().numpy().tolist() == ref["cu_seqlens"].tolist()
    assert gather.cpu().numpy()[:tot].tolist() == ref["gather_idx"].tolist()
    ga, gl = host(a_full)[:tot], host(l_full)[:tot]
    go, glo = host(a_out)[:tot], host(l_out)[:tot]
    for h in heads:
        check_a(go[:, h], ref["a_out"][:, h], f"[c5_varlen] A_out head {h}")
        check_l(glo[:, h], ref["l_out"][:, h], f"[c5_varlen] L_out head {h}")
        check_a(ga[:, h], ref["a_full"][:, h], f"[c5_varlen] A_full head {h}")
        check_l(gl[:, h], ref["l_full"][:, h], f"[c5_varlen] L_full head {h}")
    say(f"[c5_varlen] {tot} packed rows checked on all {vb.h} heads")
    # the same step through the one-launch split attention (prefix and
    # in-block parts together, then combine and merge)
    outs = {nm: torch.empty(n, vb.h, vb.d, device=dev) for nm in ("a_out", "a_in", "a_full")}
    outs.update({nm: torch.empty(n, vb.h, device=dev) for nm in ("l_out", "l_in", "l_full")})
    ba.ba_split_attn(qp, kp, vp, kb, vbk, outs["a_out"], outs["l_out"], outs["a_in"], outs["l_in"],
                     outs["a_full"], outs["l_full"], ws, q_layout="thd", kv_layout="htd", block_kv_layout="thd",
                     cu_q=cu_q, cu_kp=cu_kp, cu_k=cu_kb, max_q=max_q, max_kp=int(vb.prefix_lens.max()),
                     max_k=int(vb.block_sizes.max()))
    torch.cuda.synchronize()
    for h in heads:
        for nm in ("a_out", "a_in", "a_full"):
            check_a(host(outs[nm])[:tot, h], ref[nm][:, h], f"[c5_varlen split] {nm} head {h}")
        for nm in ("l_out", "l_in", "l_full"):
            check_l(host(outs[nm])[:tot, h], ref[nm][:, h], f"[c5_varlen split] {nm} head {h}")
    say(f"[c5_varlen] split attention checked on all {vb.h} heads")


@pytest.mark.parametrize("gate", ["count_cum", "partial"])
def test_block_graph_replays_gate_variants(gate):
    # A whole block captured as one HIP graph under the gate variants and
    # replayed three times, with unrelated eager work and synchronisation in
    # between: every replay gives the eager run's final A_full/L_full and
    # decisions bit for bit (the variants' state -- the since-refresh marks,
    # the row lists -- is rebuilt by the graph itself).
    sched = preset("c2_llada", steps=8, gate="count" if gate == "partial" else gate, tau=3)
    q, k, v = _to_dev(sched)
    kp, vp = dev_in(sched.kp, sched.dtype), dev_in(sched.vp, sched.dtype)
    attn = ba.CachedBlockAttention(kp, vp, nb=sched.nb, hq=sched.hq, gate=gate, tau=sched.tau, scale=sched.scale)
    attn.start_block()
    for t in range(1, sched.steps + 1):
        attn.step(q[t], k[t], v[t], q[t - 1], k[t - 1], v[t - 1])
    torch.cuda.synchronize()
    want = (host(attn.a_full), host(attn.l_full), attn.decision.cpu().numpy().copy())
    g = attn.capture_block(q, k, v)
    noise = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        attn.a_full.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(attn.a_full), want[0], err_msg=f"{gate} replay {rep}")
        np.testing.assert_array_equal(host(attn.l_full), want[1], err_msg=f"{gate} replay {rep}")
        assert np.array_equal(attn.decision.cpu().numpy(), want[2]), f"{gate} replay {rep}"
        noise.mul_(1.0001).add_(float(noise.sum().item()) * 0.0)
    say(f"[graph {gate}] 3 replays match the eager block")
