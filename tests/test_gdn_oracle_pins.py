"""Pins of the Gated DeltaNet scan oracle (CPU only).

Each test fixes the oracle to something other than itself: a hand-worked
example, closed forms of special cases, the delta rule's defining property,
an unrolled brute-force expansion on tiny shapes, a contraction invariant,
the head grouping and the splitting of a sequence.
"""

from __future__ import annotations

import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "gdn_worked_example.json")


def _rand(rng, T, Hk, Hv, dk, dv, unit_keys=True):
    k = rng.standard_normal((T, Hk, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = rng.standard_normal((T, Hk, dk))
    v = rng.standard_normal((T, Hv, dv))
    g = -rng.uniform(0.0, 0.7, (T, Hv))
    beta = rng.uniform(0.0, 1.0, (T, Hv))
    return q, k, v, g, beta


def test_hand_worked_example():
    d = json.load(open(GOLDEN))
    st = d["steps"]
    k = np.array([[s["k"]] for s in st])
    v = np.array([[s["v"]] for s in st])
    q = np.array([[s["q"]] for s in st])
    g = np.log(np.array([[s["alpha"]] for s in st]))
    beta = np.array([[s["beta"]] for s in st])
    o, S = oracle.gated_delta_scan(q, k, v, g, beta)
    np.testing.assert_allclose(o[:, 0, :], np.array(d["o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(S[0], np.array(d["state"]), rtol=0, atol=1e-14)


def test_no_write_is_pure_decay():
    """beta = 0: S_t = (prod of alpha up to t) S_0, o_t = S_t q_t."""
    rng = np.random.default_rng(1)
    T, Hk, Hv, dk, dv = 9, 1, 2, 5, 3
    q, k, v, g, _ = _rand(rng, T, Hk, Hv, dk, dv)
    S0 = rng.standard_normal((Hv, dv, dk))
    o, S = oracle.gated_delta_scan(q, k, v, g, np.zeros((T, Hv)), S0)
    lam = np.exp(np.cumsum(g, axis=0))          # [T][Hv]
    for t in range(T):
        for h in range(Hv):
            np.testing.assert_allclose(o[t, h], lam[t, h] * S0[h] @ q[t, 0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S, lam[-1][:, None, None] * S0, rtol=1e-12)


def test_unit_write_stores_and_replaces():
    """alpha = 1, beta = 1, unit keys: after the write S_t k_t = v_t exactly, and
    writing a key again replaces its value (the delta rule), leaving the value
    stored under an orthogonal key untouched."""
    dk, dv = 4, 3
    e = np.eye(dk)
    keys = [e[0], e[1], e[0]]
    vals = [np.array([1.0, 2.0, 3.0]), np.array([-1.0, 0.5, 4.0]), np.array([7.0, -2.0, 0.25])]
    k = np.array([[kk] for kk in keys])
    v = np.array([[vv] for vv in vals])
    q = k.copy()                                # read back the key just written
    T = len(keys)
    o, S = oracle.gated_delta_scan(q, k, v, np.zeros((T, 1)), np.ones((T, 1)))
    for t in range(T):
        np.testing.assert_array_equal(o[t, 0], vals[t])
    np.testing.assert_array_equal(S[0][:, 0], vals[2])   # replaced
    np.testing.assert_array_equal(S[0][:, 1], vals[1])   # kept
    np.testing.assert_array_equal(S[0][:, 2:], 0.0)


def test_unrolled_expansion_brute_force():
    """S_T = S_0 A_1 ... A_T + sum_t beta_t v_t k_t^T A_{t+1} ... A_T with
    A_s = alpha_s (I - beta_s k_s k_s^T), and o_t from the same expansion at t;
    dk != dv so a transposed operand cannot pass."""
    rng = np.random.default_rng(2)
    T, Hk, Hv, dk, dv = 6, 1, 1, 4, 3
    q, k, v, g, beta = _rand(rng, T, Hk, Hv, dk, dv, unit_keys=False)
    S0 = rng.standard_normal((Hv, dv, dk))
    o, S = oracle.gated_delta_scan(q, k, v, g, beta, S0)
    A = [np.exp(g[s, 0]) * (np.eye(dk) - beta[s, 0] * np.outer(k[s, 0], k[s, 0])) for s in range(T)]

    def state_at(t):                             # state after tokens 0..t
        P = np.eye(dk)
        for s in range(t + 1):
            P = P @ A[s]
        total = S0[0] @ P
        for u in range(t + 1):
            Pu = np.eye(dk)
            for s in range(u + 1, t + 1):
                Pu = Pu @ A[s]
            total = total + beta[u, 0] * np.outer(v[u, 0], k[u, 0]) @ Pu
        return total

    for t in range(T):
        np.testing.assert_allclose(o[t, 0], state_at(t) @ q[t, 0], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S[0], state_at(T - 1), rtol=1e-11, atol=1e-12)


def test_forgetting_contracts_the_state():
    """v = 0, unit keys, beta in [0, 1], alpha <= 1: every transition is a
    contraction, so the Frobenius norm of the state never grows."""
    rng = np.random.default_rng(3)
    T, Hk, Hv, dk, dv = 40, 1, 1, 6, 5
    q, k, _, g, beta = _rand(rng, T, Hk, Hv, dk, dv)
    S0 = rng.standard_normal((Hv, dv, dk))
    prev = np.linalg.norm(S0)
    S = S0
    for t in range(T):
        _, S = oracle.gated_delta_scan(q[t:t + 1], k[t:t + 1], np.zeros((1, Hv, dv)), g[t:t + 1],
                                       beta[t:t + 1], S)
        cur = np.linalg.norm(S)
        assert cur <= prev * (1 + 1e-12)
        prev = cur
    assert prev < np.linalg.norm(S0)


def test_value_heads_read_their_key_head():
    """Hk = 2, Hv = 4: value head h equals a one-head scan on key head h // 2."""
    rng = np.random.default_rng(4)
    T, Hk, Hv, dk, dv = 7, 2, 4, 5, 3
    q, k, v, g, beta = _rand(rng, T, Hk, Hv, dk, dv)
    S0 = rng.standard_normal((Hv, dv, dk))
    o, S = oracle.gated_delta_scan(q, k, v, g, beta, S0)
    for h in range(Hv):
        kh = h // 2
        o1, S1 = oracle.gated_delta_scan(q[:, kh:kh + 1], k[:, kh:kh + 1], v[:, h:h + 1],
                                         g[:, h:h + 1], beta[:, h:h + 1], S0[h:h + 1])
        np.testing.assert_array_equal(o[:, h], o1[:, 0])
        np.testing.assert_array_equal(S[h], S1[0])


def test_split_sequence_carries_the_state():
    rng = np.random.default_rng(5)
    T, Hk, Hv, dk, dv = 11, 1, 2, 4, 4
    q, k, v, g, beta = _rand(rng, T, Hk, Hv, dk, dv)
    o, S = oracle.gated_delta_scan(q, k, v, g, beta)
    oa, Sa = oracle.gated_delta_scan(q[:4], k[:4], v[:4], g[:4], beta[:4])
    ob, Sb = oracle.gated_delta_scan(q[4:], k[4:], v[4:], g[4:], beta[4:], Sa)
    np.testing.assert_array_equal(np.concatenate([oa, ob]), o)
    np.testing.assert_array_equal(Sb, S)


def test_empty_sequence_returns_the_initial_state():
    S0 = np.arange(2 * 3 * 4, dtype=np.float64).reshape(2, 3, 4)
    o, S = oracle.gated_delta_scan(np.zeros((0, 1, 4)), np.zeros((0, 1, 4)), np.zeros((0, 2, 3)),
                                   np.zeros((0, 2)), np.zeros((0, 2)), S0)
    assert o.shape == (0, 2, 3)
    np.testing.assert_array_equal(S, S0)
