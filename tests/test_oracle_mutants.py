"""CPU tests: copies of oracle functions with one planted mistake each must
fail the pins.  This shows the pins would catch such a mistake in the oracle.
"""

import numpy as np
import pytest

import oracle
from workloads import make_block_schedule
from tests import oracle_pins as pins


# --- attention mutants -------------------------------------------------------

def attn_no_max_in_lse(q, k, v, s):
    a, l = oracle.attention(q, k, v, s)
    if k.shape[0] == 0:
        return a, l
    z = s * (np.asarray(q) @ np.asarray(k).T)
    return a, l - z.max(axis=1)                       # dropped term


def attn_scale_missing(q, k, v, s):
    return oracle.attention(q, k, v, 1.0)             # scale forgotten


def attn_values_reversed(q, k, v, s):
    return oracle.attention(q, k, np.asarray(v)[::-1], s)   # wrong index


def attn_keys_for_queries(q, k, v, s):
    q = np.asarray(q)
    k = np.asarray(k)
    if k.shape[0] == 0:
        return oracle.attention(q, k, v, s)
    z = s * (q @ k.T)
    z = z - z.max(axis=0, keepdims=True)              # softmax over the wrong axis
    e = np.exp(z)
    return (e @ v) / e.sum(axis=1)[:, None], np.log(e.sum(axis=1))


@pytest.mark.parametrize("mutant", [attn_no_max_in_lse, attn_scale_missing,
                                    attn_values_reversed, attn_keys_for_queries])
def test_attention_mutants_fail(mutant):
    with pytest.raises(AssertionError):
        pins.check_attention(mutant)


# --- merge mutants -----------------------------------------------------------

def merge_wrong_sign(a1, l1, a2, l2):
    return oracle.merge(a1, -np.asarray(l1, dtype=float), a2, -np.asarray(l2, dtype=float))


def merge_no_normalise(a1, l1, a2, l2):
    a, l = oracle.merge(a1, l1, a2, l2)
    m = np.maximum(l1, l2)
    m = np.where(np.isneginf(m), 0.0, m)
    return a * np.exp(l - m)[..., None], l            # divides by nothing


def merge_lse_is_max(a1, l1, a2, l2):
    a, _ = oracle.merge(a1, l1, a2, l2)
    return a, np.maximum(l1, l2)                      # dropped log term


def merge_swapped_weights(a1, l1, a2, l2):
    a, l = oracle.merge(a1, l2, a2, l1)               # weights on the wrong side
    return a, l


@pytest.mark.parametrize("mutant", [merge_wrong_sign, merge_no_normalise,
                                    merge_lse_is_max, merge_swapped_weights])
def test_merge_mutants_fail(mutant):
    with pytest.raises(AssertionError):
        pins.check_merge(mutant, oracle.attention)


# --- gate mutants ------------------------------------------------------------

def gate_count_le(m, tau, valid, hq):
    return oracle.gate_count(np.asarray(m) - 1, tau, valid, hq)   # M <= tau


def gate_count_ignores_valid(m, tau, valid, hq):
    return oracle.gate_count(m, tau, True, hq)


def update_count_q_only(cur, prev):
    return oracle.update_count(cur[:1], prev[:1])


@pytest.mark.parametrize("gate,count", [(gate_count_le, oracle.update_count),
                                        (gate_count_ignores_valid, oracle.update_count),
                                        (oracle.gate_count, update_count_q_only)])
def test_count_gate_mutants_fail(gate, count):
    with pytest.raises(AssertionError):
        pins.check_count_gate(count, gate, make_block_schedule)


def gate_cosine_ge(cos, zero, gamma, valid):
    return oracle.gate_cosine(np.nextafter(np.asarray(cos), np.inf), zero, gamma, valid)  # >= gamma


def head_cosine_no_norm(qc, qp):
    cos, zero = oracle.head_cosine(qc, qp)
    _, z2 = oracle.head_cosine(qc, qc)
    return cos * 1.0001, zero                                     # mis-normalised


@pytest.mark.parametrize("hc,gc", [(oracle.head_cosine, gate_cosine_ge),
                                   (head_cosine_no_norm, oracle.gate_cosine)])
def test_cosine_gate_mutants_fail(hc, gc):
    with pytest.raises(AssertionError):
        pins.check_cosine_gate(hc, gc)


# --- packing mutants ---------------------------------------------------------

def pack_inclusive(locked, bs):
    cu, g, t = oracle.varlen_pack(locked, bs)
    return np.concatenate([cu[1:], cu[-1:]]), g, t


def pack_counts_locked(locked, bs):
    return oracle.varlen_pack(1 - np.asarray(locked), bs)


def pack_reversed(locked, bs):
    cu, g, t = oracle.varlen_pack(locked, bs)
    g = g.copy()
    for b in range(len(bs)):
        g[cu[b]:cu[b + 1]] = g[cu[b]:cu[b + 1]][::-1]
    return cu, g, t


@pytest.mark.parametrize("mutant", [pack_inclusive, pack_counts_locked, pack_reversed])
def test_pack_mutants_fail(mutant):
    with pytest.raises(AssertionError):
        pins.check_pack(mutant)


# --- cumulative count gate mutants ------------------------------------------

def cum_never_restarts(changed, tau, hq):
    # counts from step 1 whatever the refreshes
    out = [None]
    union = None
    for t in range(1, len(changed)):
        union = changed[t].copy() if union is None else union | changed[t]
        m = union.sum(axis=1).astype(np.int32)
        out.append(dict(m=m, decision=oracle.gate_count(m, tau, t > 1, hq)))
    return out


def cum_includes_refresh_step(changed, tau, hq):
    # the union also takes the refresh step's own updates (off by one)
    out = [None]
    for t in range(1, len(changed)):
        B = changed[t].shape[0]
        m = np.zeros(B, dtype=np.int32)
        for b in range(B):
            r = 0
            for s_ in range(1, t):
                if out[s_]["decision"][b, 0] == 0:
                    r = s_
            union = np.zeros(changed[t].shape[1], dtype=bool)
            for s_ in range(max(r, 1), t + 1):
                union |= changed[s_][b]
            m[b] = int(union.sum())
        out.append(dict(m=m, decision=oracle.gate_count(m, tau, t > 1, hq)))
    return out


def cum_tie_reuses(changed, tau, hq):
    return oracle.cumulative_gates(changed, tau + 1, hq)   # reuse iff M <= tau


def cum_per_step(changed, tau, hq):
    out = [None]
    for t in range(1, len(changed)):
        m = changed[t].sum(axis=1).astype(np.int32)
        out.append(dict(m=m, decision=oracle.gate_count(m, tau, t > 1, hq)))
    return out


@pytest.mark.parametrize("mutant", [cum_never_restarts, cum_includes_refresh_step, cum_tie_reuses, cum_per_step])
def test_cumulative_gate_mutants_fail(mutant):
    with pytest.raises(AssertionError):
        pins.check_cumulative_gate(mutant)


def rows_first_head_only(q_cur, q_prev):
    return oracle.rows_changed(np.asarray(q_cur)[:, :, :1], np.asarray(q_prev)[:, :, :1])


def rows_by_value(q_cur, q_prev):
    # compares values after a lossy float conversion instead of bits
    return (np.asarray(q_cur).astype(np.float16) != np.asarray(q_prev).astype(np.float16)).any(axis=(2, 3))


@pytest.mark.parametrize("mutant", [rows_first_head_only, rows_by_value])
def test_rows_changed_mutants_fail(mutant):
    with pytest.raises(AssertionError):
        pins.check_rows_changed(mutant)
