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
