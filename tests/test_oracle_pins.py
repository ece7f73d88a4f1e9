"""Pins of the CPU oracle against facts fixed outside it.

Each test checks the oracle against something it does not compute itself:
exact rational arithmetic, brute-force enumeration, closed forms, library
routines, invariants, and the figures printed on the pages (tests/golden).
A plausible slip in the oracle (a dropped term, a swapped operand, a wrong
nibble, a sign, an off-by-one in a table) fails at least one of them.
"""

from __future__ import annotations

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from synth import (FULL_SHAPE, bf16_bits_to_f32, build_config, f64_to_bf16_bits, make_bank,
                   make_router, make_tokens)
from synth.configs import bank_nbytes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- exact helpers

def rne(fr: Fraction, p: int) -> Fraction:
    """Round a rational to p significant bits, ties to even (normal range)."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - (p - 1))
    scaled = a / ulp
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def f32(v) -> Fraction:
    return Fraction(float(np.float32(v)))


def np_dequant(q, s, b):
    """Independent reconstruction: unpack nibbles, q*s+b exactly in float64, round
    to float32 (numpy RNE), then to bfloat16 (frexp-based RNE of the generator)."""
    q = np.asarray(q)
    rows, half = q.shape
    codes = np.empty((rows, 2 * half), dtype=np.float64)
    codes[:, 0::2] = q & 0x0F
    codes[:, 1::2] = q >> 4
    sf = np.repeat(bf16_bits_to_f32(s).astype(np.float64), 64, axis=1)
    bf = np.repeat(bf16_bits_to_f32(b).astype(np.float64), 64, axis=1)
    w = (codes * sf + bf).astype(np.float32).astype(np.float64)
    return bf16_bits_to_f32(f64_to_bf16_bits(w)).astype(np.float64)


def silu(z):
    return z / (1.0 + np.exp(-z))


# ---------------------------------------------------------------- page facts

def test_page_facts_format_size():
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    g = facts["quant_group"]["value"]
    bits = facts["code_bits"]["value"] + 2 * facts["scale_bias_bits"]["value"] / g
    assert bits == 4.5
    # one expert of the full shape: 3*H*I weights at 4.5 bits each
    assert bank_nbytes(FULL_SHAPE) * 8 == 3 * FULL_SHAPE.H * FULL_SHAPE.I * bits
    # 70 GB of bf16 at 4.5 bits/weight is within 2% of the printed 19.4 GB
    expect = facts["bf16_checkpoint_gb"]["value"] * bits / 16
    assert abs(expect - facts["w4_checkpoint_gb"]["value"]) / facts["w4_checkpoint_gb"]["value"] < 0.02
    assert FULL_SHAPE.E == facts["routed_experts"]["value"]
    assert FULL_SHAPE.k == facts["selected_experts"]["value"]
    assert FULL_SHAPE.n_shared == facts["shared_experts"]["value"]


# ---------------------------------------------------------------- bfloat16 rounding

def test_bf16_rne_ties_and_agreement(orc):
    one = 1.0
    cases = [
        (one + 2.0 ** -8, 0x3F80),              # tie, even neighbour is 1.0
        (one + 3 * 2.0 ** -8, 0x3F82),          # tie, rounds up to even
        (one + 2.0 ** -8 + 2.0 ** -20, 0x3F81),  # above the tie
        (-(one + 2.0 ** -8), 0xBF80),
        (0.0, 0x0000),
        (-0.0, 0x8000),
    ]
    for v, bits in cases:
        assert int(orc.f32_to_bf16(np.float32(v))[0]) == bits, v
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    a = orc.f32_to_bf16(v)
    b = f64_to_bf16_bits(v.astype(np.float64))
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- dequantisation

def test_dequant_closed_forms(orc):
    K = 64
    # scale 1, bias 0: the weight is the code itself; checks nibble order too
    q = np.array([[(2 * i + 1) % 16 << 4 | (2 * i) % 16 for i in range(K // 2)]], dtype=np.uint8)
    one = f64_to_bf16_bits(np.array([[1.0]]))
    zero = f64_to_bf16_bits(np.array([[0.0]]))
    w = orc.dequant(q, one, zero)
    assert np.array_equal(w[0], np.arange(K, dtype=np.float32) % 16)
    # code 8 with bias -8*scale reconstructs to exactly zero
    s = f64_to_bf16_bits(np.array([[0.0137]]))
    b = f64_to_bf16_bits(-8.0 * bf16_bits_to_f32(s).astype(np.float64))
    w = orc.dequant(np.full((1, K // 2), 0x88, dtype=np.uint8), s, b)
    assert np.all(w == 0.0)


def test_dequant_single_rounding_exact(orc):
    """Every code of many groups against exact rational arithmetic."""
    rng = np.random.default_rng(1)
    n_groups = 40
    s = f64_to_bf16_bits(rng.uniform(0.002, 0.02, (n_groups, 1)))
    b = f64_to_bf16_bits(-8.0 * bf16_bits_to_f32(s).astype(np.float64))
    b[::3] = f64_to_bf16_bits(rng.uniform(-0.2, 0.2, (len(b[::3]), 1)))  # general biases too
    codes = np.tile(np.arange(16), 4)
    q = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    q = np.tile(q, (n_groups, 1))
    w = orc.dequant(q, s, b)
    n_rounded = 0
    for g in range(n_groups):
        sf = Fraction(float(bf16_bits_to_f32(s[g, 0])))
        bf = Fraction(float(bf16_bits_to_f32(b[g, 0])))
        for kk in range(64):
            exact = codes[kk] * sf + bf
            want = rne(rne(exact, 24), 8)
            assert Fraction(float(w[g, kk])) == want, (g, kk)
            n_rounded += want != exact
    assert n_rounded > 100   # the reconstruction really does round


def test_dequant_matches_independent_unpack(orc):
    bank = make_bank(2, 128, 64, seed=5, prefix="pin")
    for part in ("gu", "dn"):
        for e in range(2):
            a = orc.dequant(bank[f"{part}_q"][e], bank[f"{part}_s"][e], bank[f"{part}_b"][e])
            ref = np_dequant(bank[f"{part}_q"][e], bank[f"{part}_s"][e], bank[f"{part}_b"][e])
            assert np.array_equal(a.astype(np.float64), ref)


# ---------------------------------------------------------------- router logits

def test_logits_exact_on_integer_inputs(orc):
    rng = np.random.default_rng(2)
    T, H, E = 5, 256, 7
    xi = rng.integers(-8, 9, (T, H))
    wi = rng.integers(-8, 9, (H, E))
    bi = rng.integers(-50, 51, E)
    x = f64_to_bf16_bits(xi.astype(np.float64))
    l = orc.router_logits(x, wi.astype(np.float32), bi.astype(np.float32))
    assert np.array_equal(l.astype(np.int64), xi @ wi + bi)
    l0 = orc.router_logits(x, wi.astype(np.float32), None)
    assert np.array_equal(l0.astype(np.int64), xi @ wi)


def test_logits_within_float32_error_bound(orc):
    c = build_config("prefill512", T=16, with_weights=False)
    x, wr = c["x"], c["wr"]
    bias = np.linspace(-1, 1, wr.shape[1]).astype(np.float32)
    l32 = orc.router_logits(x, wr, bias).astype(np.float64)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    wf = wr.astype(np.float64)
    exact = xf @ wf + bias
    mag = np.abs(xf) @ np.abs(wf) + np.abs(bias)
    H = x.shape[1]
    bound = (H // 64 + 8) * 2.0 ** -24 * mag
    assert np.all(np.abs(l32 - exact) <= bound)
    l64 = orc.router_logits_f64(x, wr, bias)
    assert np.allclose(l64, exact, rtol=0, atol=1e-12)


def test_logits_order_exact_rational(orc):
    """The fixed order (64 strided fma chains, then the pairwise tree) emulated exactly."""
    rng = np.random.default_rng(3)
    T, H, E = 2, 128, 2
    x = f64_to_bf16_bits(rng.standard_normal((T, H)) * np.exp(rng.uniform(-6, 6, (T, H))))
    wr = (rng.standard_normal((H, E)) * np.exp(rng.uniform(-6, 6, (H, E)))).astype(np.float32)
    bias = rng.standard_normal(E).astype(np.float32)
    got = orc.router_logits(x, wr, bias)
    xf = bf16_bits_to_f32(x)
    seq_differs = 0
    for t in range(T):
        for e in range(E):
            p = []
            for m in range(64):
                acc = Fraction(0)
                for h in range(m, H, 64):
                    acc = rne(Fraction(float(xf[t, h])) * f32(wr[h, e]) + acc, 24)
                p.append(acc)
            s = 32
            while s >= 1:
                for i in range(s):
                    p[i] = rne(p[i] + p[i + s], 24)
                s //= 2
            want = rne(p[0] + f32(bias[e]), 24)
            assert Fraction(float(got[t, e])) == want
            seq = Fraction(0)
            for h in range(H):
                seq = rne(Fraction(float(xf[t, h])) * f32(wr[h, e]) + seq, 24)
            seq_differs += rne(seq + f32(bias[e]), 24) != want
    assert seq_differs >= 1   # the order is not a plain left-to-right chain


# ---------------------------------------------------------------- top-k and weights

def test_topk_brute_force(orc):
    rng = np.random.default_rng(4)
    E = 7
    for k in range(1, E + 1):
        logits = rng.standard_normal((6, E)).astype(np.float32)
        idx, w = orc.topk(logits, k)
        for t in range(6):
            best = max(itertools.combinations(range(E), k), key=lambda S: sum(float(logits[t, e]) for e in S))
            assert sorted(idx[t]) == sorted(best)
            assert all(logits[t, idx[t, j]] >= logits[t, idx[t, j + 1]] for j in range(k - 1))
            p = np.exp(logits[t].astype(np.float64) - logits[t].max())
            p /= p.sum()
            ref = p[idx[t]] / p[idx[t]].sum()
            assert np.allclose(w[t], ref, rtol=1e-14, atol=0)
            assert abs(w[t].sum() - 1.0) < 1e-14


def test_topk_special_cases_and_ties(orc):
    logits = np.array([[0.5, 2.0, 2.0, -1.0, 2.0, 0.0]], dtype=np.float32)
    idx, w = orc.topk(logits, 2)
    assert idx.tolist() == [[1, 2]]              # equal logits: lower index first
    assert np.allclose(w, 0.5)
    idx, w = orc.topk(logits, 1)
    assert idx.tolist() == [[1]] and w[0, 0] == 1.0   # k=1: argmax, weight one
    idx, w = orc.topk(logits, 6)                 # k=E: full order, weights = softmax
    assert idx.tolist() == [[1, 2, 4, 0, 5, 3]]
    from scipy.special import softmax
    assert np.allclose(w[0], softmax(logits[0].astype(np.float64))[idx[0]], rtol=1e-14)
    z = np.array([[0.0, -0.0, 0.0]], dtype=np.float32)   # signed zeros compare equal
    assert orc.topk(z, 2)[0].tolist() == [[0, 1]]


# ---------------------------------------------------------------- histogram / scan / scatter

def test_route_tables_invariants_and_brute_force(orc):
    rng = np.random.default_rng(5)
    for T, E, k in ((1, 4, 2), (13, 8, 3), (64, 16, 4), (200, 256, 8)):
        idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        counts, offsets, ss, sp = orc.route_tables(idx, E)
        assert counts.sum() == T * k
        assert offsets[0] == 0 and offsets[E] == T * k
        assert np.all(np.diff(offsets) == counts)
        assert np.array_equal(np.sort(ss), np.arange(T * k))
        assert np.array_equal(sp[ss], np.arange(T * k))
        flat = idx.ravel()
        brute = [s for e in range(E) for s in range(T * k) if flat[s] == e]
        assert ss.tolist() == brute
        assert np.array_equal(ss, np.argsort(flat, kind="stable"))
        for e in range(E):
            assert np.all(flat[ss[offsets[e]:offsets[e + 1]]] == e)


# ---------------------------------------------------------------- block map

def check_block_map(blocks, counts, offsets, T, k, E, n_shared, M, gran):
    groups = {}
    for g, r0, rows, tm in blocks.tolist():
        groups.setdefault(g, []).append((r0, rows, tm))
        assert 1 <= rows <= tm <= M and tm % gran == 0
    assert [b[0] for b in blocks.tolist()] == sorted(b[0] for b in blocks.tolist())
    for g in range(E + n_shared):
        c = int(counts[g]) if g < E else T
        first = int(offsets[g]) if g < E else T * k
        bl = groups.get(g, [])
        if c == 0:
            assert not bl
            continue
        assert len(bl) == math.ceil(c / M)
        assert sum(r for _, r, _ in bl) == c
        assert max(r for _, r, _ in bl) - min(r for _, r, _ in bl) <= 1
        assert [r for _, r, _ in bl] == sorted((r for _, r, _ in bl), reverse=True)
        row = first
        for r0, rows, tm in bl:
            assert r0 == row
            row += rows
            assert tm == -(-max(r for _, r, _ in bl) // gran) * gran


def test_block_map_rule(orc):
    rng = np.random.default_rng(6)
    for T, E, k, n_shared, M, gran in ((16, 8, 2, 1, 128, 16), (300, 16, 4, 1, 32, 16),
                                        (2048, 64, 8, 1, 128, 16), (5, 8, 8, 0, 16, 16),
                                        (777, 32, 3, 1, 256, 32)):
        p = rng.dirichlet(np.full(E, 0.3))
        idx = np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
        counts, offsets, _, _ = orc.route_tables(idx, E)
        blocks = orc.block_map(T, E, k, n_shared, M, gran, counts, offsets)
        check_block_map(blocks, counts, offsets, T, k, E, n_shared, M, gran)
        assert len(blocks) <= orc.max_blocks(T, E, k, n_shared, M)
    # the worked cases of the rule: 300 rows at M=128 -> 3 blocks of 100, tile 112
    counts = np.array([300, 0, 1], dtype=np.int32)
    offsets = np.array([0, 300, 300, 301], dtype=np.int32)
    bl = orc.block_map(301, 3, 1, 0, 128, 16, counts, offsets)
    assert bl.tolist() == [[0, 0, 100, 112], [0, 100, 100, 112], [0, 200, 100, 112], [2, 300, 1, 16]]


# ---------------------------------------------------------------- expert FFN and layer

def dense_reference(x, routed, shared, idx, w):
    """numpy float64 layer from independently reconstructed weights."""
    xf = bf16_bits_to_f32(x).astype(np.float64)
    E = routed["gu_q"].shape[0]
    I = routed["gu_q"].shape[1] // 2

    def ffn(bank, e):
        gu = np_dequant(bank["gu_q"][e], bank["gu_s"][e], bank["gu_b"][e])
        dn = np_dequant(bank["dn_q"][e], bank["dn_s"][e], bank["dn_b"][e])
        g = xf @ gu[:I].T
        u = xf @ gu[I:].T
        return (silu(g) * u) @ dn.T        # every token through this expert

    dense = np.stack([ffn(routed, e) for e in range(E)])      # [E][T][H]
    T = x.shape[0]
    y = np.zeros((T, x.shape[1]))
    for t in range(T):
        for j in range(idx.shape[1]):
            y[t] += w[t, j] * dense[idx[t, j], t]
    if shared is not None:
        y += ffn(shared, 0)
    return y


def test_layer_dense_brute_force_tiny(orc):
    c = build_config("tiny16")
    r = orc.route(c["x"], c["wr"], c["bias"], 2, 1, 128, 16)
    y = orc.moe_layer(c["x"], r["topk_idx"], r["topk_w"], c["routed"], c["shared"])
    ref = dense_reference(c["x"], c["routed"], c["shared"], r["topk_idx"], r["topk_w"])
    assert np.allclose(y, ref, rtol=1e-11, atol=1e-12)


def test_single_expert_reduces_to_dense_swiglu(orc):
    H, I = 128, 64
    bank = make_bank(1, H, I, seed=7, prefix="dense")
    x = make_tokens(3, H, seed=7)
    idx = np.zeros((3, 1), dtype=np.int32)
    w = np.ones((3, 1))
    y = orc.moe_layer(x, idx, w, bank, None)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    gu = np_dequant(bank["gu_q"][0], bank["gu_s"][0], bank["gu_b"][0])
    dn = np_dequant(bank["dn_q"][0], bank["dn_s"][0], bank["dn_b"][0])
    ref = (silu(xf @ gu[:I].T) * (xf @ gu[I:].T)) @ dn.T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-13)
    h, y1 = orc.expert_ffn(x[1], bank, 0)
    assert np.allclose(h, (silu(xf @ gu[:I].T) * (xf @ gu[I:].T))[1], rtol=1e-12, atol=1e-14)
    assert np.allclose(y1, ref[1], rtol=1e-12, atol=1e-13)


def test_zero_cases(orc):
    H, I = 128, 64
    bank = make_bank(2, H, I, seed=8, prefix="zero")
    x = make_tokens(4, H, seed=8)
    idx = np.array([[0, 1]] * 4, dtype=np.int32)
    w = np.full((4, 2), 0.5)
    zb = {kk: v.copy() for kk, v in bank.items()}
    zb["gu_q"][:, :I] = 0x88       # gate weights all reconstruct to zero
    assert np.all(orc.moe_layer(x, idx, w, zb, None) == 0.0)
    zb = {kk: v.copy() for kk, v in bank.items()}
    zb["gu_q"][:, I:] = 0x88       # up weights all zero
    assert np.all(orc.moe_layer(x, idx, w, zb, None) == 0.0)
    x0 = np.zeros_like(x)
    assert np.all(orc.moe_layer(x0, idx, w, bank, {kk: v[:1] for kk, v in bank.items()}) == 0.0)


def test_equivariances(orc):
    c = build_config("tiny16")
    x, wr = c["x"], c["wr"]
    r = orc.route(x, wr, None, 2, 1, 128, 16)
    y = orc.moe_layer(x, r["topk_idx"], r["topk_w"], c["routed"], c["shared"])
    # token permutation
    perm = np.random.default_rng(9).permutation(x.shape[0])
    rp = orc.route(x[perm], wr, None, 2, 1, 128, 16)
    yp = orc.moe_layer(x[perm], rp["topk_idx"], rp["topk_w"], c["routed"], c["shared"])
    assert np.array_equal(yp, y[perm])
    # expert relabelling: permute router columns and banks together
    E = wr.shape[1]
    pe = np.random.default_rng(10).permutation(E)
    routed_p = {kk: v[pe] for kk, v in c["routed"].items()}
    rr = orc.route(x, wr[:, pe], None, 2, 1, 128, 16)
    yr = orc.moe_layer(x, rr["topk_idx"], rr["topk_w"], routed_p, c["shared"])
    assert np.array_equal(pe[rr["topk_idx"]], r["topk_idx"])
    assert np.allclose(yr, y, rtol=1e-14, atol=1e-15)


def test_zipf_config_reading(orc):
    """The skewed router leaves experts empty and overloads a few (the point of that workload)."""
    c = build_config("prefill2048_zipf", with_weights=False)
    r = orc.route(c["x"], c["wr"], c["bias"], 8, 1, 128, 16)
    counts = r["counts"]
    assert (counts == 0).sum() >= 1 and (counts > 200).sum() >= 1
    check_block_map(r["blocks"], counts, r["offsets"], 2048, 8, 256, 1, 128, 16)
    w = r["topk_w"]
    assert np.all(np.abs(w.sum(1) - 1.0) < 1e-12)


def test_router_init_scale():
    wr = make_router(2048, 256, 0.02, seed=1)
    assert abs(wr.std() - 0.02) < 2e-4 and abs(wr.mean()) < 2e-4


# ---------------------------------------------------------------- the output metrics

def test_relative_error_metrics_hand_computed(orc):
    """Both layer-output metrics on arrays worked out by hand: a zero reference
    row (its denominator falls back to 1), and a worst token that is not the
    first one."""
    y_ref = np.array([[1.0, -2.0, 0.5],
                      [0.0, 0.0, 0.0],
                      [4.0, 1.0, -1.0]])
    delta = np.array([[0.01, 0.0, 0.0],
                      [0.001, 0.0, 0.0],
                      [0.0, 0.1, 0.0]])
    y = y_ref + delta
    # normwise, per token max_i |dy| / max_i |y_ref|: 0.01/2, 0.001/1, 0.1/4
    assert orc.relative_error(y, y_ref) == pytest.approx(0.025, rel=1e-12)
    assert orc.relative_error(y[:2], y_ref[:2]) == pytest.approx(0.005, rel=1e-12)
    # elementwise, |dy| / max(|y_ref|, rms of the token's row):
    # row 0: 0.01 / max(1, sqrt(5.25/3)); row 1: 0.001 / 1; row 2: 0.1 / max(1, sqrt(18/3))
    assert orc.relative_error_elementwise(y, y_ref) == pytest.approx(0.1 / math.sqrt(6.0), rel=1e-12)
    assert orc.relative_error_elementwise(y[:1], y_ref[:1]) == pytest.approx(0.01 / math.sqrt(1.75),
                                                                            rel=1e-12)
    # an element larger than its row's rms is measured against itself
    assert orc.relative_error_elementwise(np.array([[10.5, 0.0, 0.0, 0.0]]),
                                          np.array([[10.0, 0.0, 0.0, 0.0]])) == pytest.approx(0.05)
    # symmetric in the sign of the error, exact on equality, empty is zero
    assert orc.relative_error(y_ref - delta, y_ref) == pytest.approx(0.025, rel=1e-12)
    assert orc.relative_error(y_ref, y_ref) == 0.0 == orc.relative_error_elementwise(y_ref, y_ref)
    assert orc.relative_error(np.zeros((0, 3)), np.zeros((0, 3))) == 0.0
