"""Pins of the CPU oracle to things other than itself (CPU only).

Each check is a function of an oracle implementation ``o`` so the same checks can
be run against deliberately broken copies of the oracle (see
test_oracle_mutants.py): a plausible slip in the oracle must fail at least one.

Pins used (the pages print no worked numbers):
* hand-derived block values (tests/golden/q8_hand_blocks.txt);
* exact rational brute force on tiny random shapes (fractions.Fraction);
* closed forms and invariants: linearity in d and in x, zero-scale blocks, one-hot
  gathers, sign symmetry;
* library routines for special cases: scipy's expit (SiLU), scipy's softmax
  (top-k with k = E), Python's sorted() (top-k selection);
* the MoE mixture reducing to one dense SwiGLU FFN (k = 1, identical experts) and
  invariance under relabelling the experts.
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import oracle as O
import workloads as wl
from golden_io import (half_bits_to_fraction, load_act_quant_cases, load_k_quant_cases, load_linear_cases,
                       load_q4_0_cases, load_swiglu_router_cases)

LINEAR_CASES = load_linear_cases()
FUSED_CASES, ROUTE_CASES = load_swiglu_router_cases()
ACT_CASES = load_act_quant_cases()
Q4_CASES = load_q4_0_cases()
KQ_CASES = load_k_quant_cases()


# ------------------------------------------------------------------ checks


def check_hand_linear(o):
    for c in LINEAR_CASES:
        y = o.q8_linear_ref(c["w"], c["n"], c["k"], np.array(c["x"]))
        want = np.array([[float(v) for v in r] for r in c["y"]])
        assert y.shape == want.shape, c["name"]
        # every case is exact in float64
        for got, exp in zip(y.ravel(), [v for r in c["y"] for v in r]):
            assert Fraction(float(got)) == exp, (c["name"], float(got), exp)


def check_hand_fused(o):
    for c in FUSED_CASES:
        h = o.fused_gate_up_silu_ref(c["w"], 1, c["k"], np.array(c["x"]))
        assert h.shape == (1, 1)
        assert math.isclose(float(h[0, 0]), c["h"], rel_tol=1e-14, abs_tol=1e-300), c["name"]


def check_hand_route(o):
    for c in ROUTE_CASES:
        idx, w = o.route_topk_ref(np.array(c["x"]), np.array(c["w_router"]), c["k"], c["normalize"])
        assert idx.tolist() == c["idx"], c["name"]
        np.testing.assert_allclose(w, np.array(c["w"]), rtol=1e-14, atol=0, err_msg=c["name"])


def _exact_linear(q, d, x):
    """Fraction brute force: y[m][n] = sum_k x[m][k] * d[n][k//32] * q[n][k]."""
    n, k = q.shape
    m = x.shape[0]
    dq = [[half_bits_to_fraction(int(b)) for b in row] for row in d.view(np.uint16)]
    xf = [[Fraction(float(v)) for v in row] for row in x]
    out = [[Fraction(0)] * n for _ in range(m)]
    for mi in range(m):
        for ni in range(n):
            s = Fraction(0)
            for ki in range(k):
                s += xf[mi][ki] * dq[ni][ki // 32] * int(q[ni, ki])
            out[mi][ni] = s
    return out


def check_bruteforce_linear(o):
    for seed, (n, k, m) in enumerate([(1, 32, 1), (3, 64, 2), (2, 256, 1), (3, 96, 2)]):
        wb, q, d = wl.q8_weight(100 + seed, n, k)
        x = wl.activations(200 + seed, m, k)
        y = o.q8_linear_ref(wb, n, k, x)
        ex = _exact_linear(q, d, x)
        for mi in range(m):
            for ni in range(n):
                e = float(ex[mi][ni])
                assert abs(y[mi, ni] - e) <= 1e-12 * max(1.0, abs(e)), (n, k, m, mi, ni)


def check_dequant_exact(o):
    wb, q, d = wl.q8_weight(7, 3, 128)
    w = o.dequantize_q8_0(wb, 3, 128)
    dq = d.view(np.uint16)
    for n in range(3):
        for kk in range(128):
            assert Fraction(float(w[n, kk])) == half_bits_to_fraction(int(dq[n, kk // 32])) * int(q[n, kk])


def check_linearity(o):
    n, k, m = 5, 256, 3
    _, q, d = wl.q8_weight(11, n, k)
    x = wl.activations(12, m, k)
    y = o.q8_linear_ref(wl.pack_blocks(q, d), n, k, x)
    # doubling every scale doubles y exactly (power of two; no binary16 overflow here)
    y2 = o.q8_linear_ref(wl.pack_blocks(q, (d.astype(np.float32) * 2).astype(np.float16)), n, k, x)
    assert np.array_equal(y2, 2 * y)
    # y(2x) = 2 y(x) exactly
    assert np.array_equal(o.q8_linear_ref(wl.pack_blocks(q, d), n, k, 2 * x), 2 * y)
    # additivity in x
    x2 = wl.activations(13, m, k)
    ya = o.q8_linear_ref(wl.pack_blocks(q, d), n, k, x.astype(np.float64) + x2)
    yb = y + o.q8_linear_ref(wl.pack_blocks(q, d), n, k, x2)
    np.testing.assert_allclose(ya, yb, rtol=1e-12, atol=1e-12)
    # sign symmetry q -> -q (no -128 in the draw)
    yneg = o.q8_linear_ref(wl.pack_blocks(-q, d), n, k, x)
    assert np.array_equal(yneg, -y)


def check_zero_scale(o):
    n, k, m = 4, 256, 2
    _, q, d = wl.q8_weight(21, n, k)
    x = wl.activations(22, m, k)
    rng = np.random.default_rng(5)
    mask = rng.random(d.shape) < 0.4
    d0 = d.copy()
    d0[mask] = 0
    q0 = q.copy().reshape(n, k // 32, 32)
    q0[mask] = 0
    ya = o.q8_linear_ref(wl.pack_blocks(q, d0), n, k, x)
    yb = o.q8_linear_ref(wl.pack_blocks(q0.reshape(n, k), d), n, k, x)
    np.testing.assert_allclose(ya, yb, rtol=1e-13, atol=1e-13)
    yz = o.q8_linear_ref(wl.pack_blocks(q, np.zeros_like(d)), n, k, x)
    assert np.all(yz == 0)


def check_one_hot(o):
    n, k, m = 6, 128, 3
    perm = np.random.default_rng(3).permutation(k)[:n]
    q = np.zeros((n, k), np.int8)
    q[np.arange(n), perm] = 1
    d = np.ones((n, k // 32), np.float16)
    x = wl.activations(31, m, k)
    y = o.q8_linear_ref(wl.pack_blocks(q, d), n, k, x)
    assert np.array_equal(y, x[:, perm].astype(np.float64))


def check_silu(o):
    g = np.linspace(-40, 40, 2001)
    np.testing.assert_allclose(o.silu_ref(g), g * scipy.special.expit(g), rtol=1e-14, atol=1e-300)
    # silu(g) - silu(-g) = g
    np.testing.assert_allclose(o.silu_ref(g) - o.silu_ref(-g), g, rtol=1e-13, atol=1e-13)
    assert o.silu_ref(np.array([0.0]))[0] == 0.0
    assert np.all(np.isfinite(o.silu_ref(np.array([-800.0, 800.0]))))


def check_fused_split(o):
    """gate rows [0,F), up rows [F,2F): the fused result equals two plain linears."""
    f, k, m = 8, 256, 2
    _, qg, dg = wl.q8_weight(41, f, k)
    _, qu, du = wl.q8_weight(42, f, k)
    x = wl.activations(43, m, k)
    g = o.q8_linear_ref(wl.pack_blocks(qg, dg), f, k, x)
    u = o.q8_linear_ref(wl.pack_blocks(qu, du), f, k, x)
    fused = wl.pack_blocks(np.concatenate([qg, qu]), np.concatenate([dg, du]))
    h = o.fused_gate_up_silu_ref(fused, f, k, x)
    np.testing.assert_allclose(h, g * scipy.special.expit(g) * u, rtol=1e-13, atol=1e-13)


def _sorted_topk(p_row, k):
    order = sorted(range(len(p_row)), key=lambda e: (-p_row[e], e))
    return order[:k]


def check_route_invariants(o):
    m, h, e = 6, 64, 16
    x = wl.activations(51, m, h)
    wr = wl.router_weight(52, e, h, std=0.5)
    logits = x.astype(np.float64) @ wr.astype(np.float64).T
    p_lib = scipy.special.softmax(logits, axis=-1)
    for k in (1, 3, e):
        idx, w = o.route_topk_ref(x, wr, k, True)
        idx_raw, w_raw = o.route_topk_ref(x, wr, k, False)
        assert np.array_equal(idx, idx_raw)
        for mi in range(m):
            assert idx[mi].tolist() == _sorted_topk(list(p_lib[mi]), k)
            # renormalized weights = softmax over the selected logits
            sel = logits[mi, idx[mi]]
            np.testing.assert_allclose(w[mi], scipy.special.softmax(sel), rtol=1e-12)
            assert abs(w[mi].sum() - 1.0) < 1e-14
            np.testing.assert_allclose(w_raw[mi], p_lib[mi, idx[mi]], rtol=1e-12)
            assert np.all(np.diff(w[mi]) <= 0)
        if k == e:
            np.testing.assert_allclose(np.take_along_axis(p_lib, idx.astype(np.int64), 1), w, rtol=1e-12)


def _dense_ffn(o, gu, dn, f, h, x):
    hid = o.fused_gate_up_silu_ref(gu, f, h, x)
    return o.q8_linear_ref(dn, h, f, hid)


def _stack(parts):
    return np.concatenate([np.asarray(p, np.uint8) for p in parts])


def check_moe(o):
    e_n, f, h, m, k = 4, 64, 64, 3, 2
    gus = [wl.q8_weight(60 + i, 2 * f, h) for i in range(e_n)]
    dns = [wl.q8_weight(70 + i, h, f) for i in range(e_n)]
    gu_stack = _stack([g[0] for g in gus])
    dn_stack = _stack([d[0] for d in dns])
    x = wl.activations(80, m, h)
    # k = 1, weight 1: one dense SwiGLU FFN of the chosen expert
    idx = np.array([[2], [0], [3]], np.int32)
    w1 = np.ones((m, 1))
    y = o.moe_mixture_ref(gu_stack, dn_stack, e_n, f, h, x, idx, w1)
    for mi in range(m):
        e = int(idx[mi, 0])
        want = _dense_ffn(o, gus[e][0], dns[e][0], f, h, x[mi:mi + 1])[0]
        np.testing.assert_allclose(y[mi], want, rtol=1e-13, atol=1e-13)
    # general k: explicit weighted sum of dense FFNs, slot order
    idx, wts = wl.random_routing(81, m, e_n, k)
    y = o.moe_mixture_ref(gu_stack, dn_stack, e_n, f, h, x, idx, wts)
    for mi in range(m):
        want = np.zeros(h)
        for j in range(k):
            e = int(idx[mi, j])
            want += float(wts[mi, j]) * _dense_ffn(o, gus[e][0], dns[e][0], f, h, x[mi:mi + 1])[0]
        np.testing.assert_allclose(y[mi], want, rtol=1e-12, atol=1e-12)
    # identical experts + renormalized routing = one FFN
    same_gu = _stack([gus[0][0]] * e_n)
    same_dn = _stack([dns[0][0]] * e_n)
    wr = wl.router_weight(82, e_n, h, std=0.3)
    ys, _, _ = o.moe_ref(wr, same_gu, same_dn, e_n, f, h, x, k, True)
    np.testing.assert_allclose(ys, _dense_ffn(o, gus[0][0], dns[0][0], f, h, x), rtol=1e-12, atol=1e-12)
    # relabelling experts (router rows with the stacks) leaves y unchanged
    perm = np.array([2, 0, 3, 1])
    ya, _, _ = o.moe_ref(wr, gu_stack, dn_stack, e_n, f, h, x, k, True)
    yb, _, _ = o.moe_ref(wr[perm], _stack([gus[p][0] for p in perm]), _stack([dns[p][0] for p in perm]),
                         e_n, f, h, x, k, True)
    np.testing.assert_allclose(ya, yb, rtol=1e-13, atol=1e-13)


def check_moe_bruteforce(o):
    """Pure-Python loops over every index (tiny shapes, math.exp), from generator q/d."""
    e_n, f, h, m, k = 3, 32, 32, 2, 2
    gus = [wl.q8_weight(90 + i, 2 * f, h) for i in range(e_n)]
    dns = [wl.q8_weight(95 + i, h, f) for i in range(e_n)]
    x = wl.activations(99, m, h)
    idx, wts = wl.random_routing(98, m, e_n, k)
    y = o.moe_mixture_ref(_stack([g[0] for g in gus]), _stack([d[0] for d in dns]), e_n, f, h, x, idx, wts)

    def wval(qd, r, c):
        _, q, d = qd
        return float(d[r, c // 32]) * int(q[r, c])

    for mi in range(m):
        acc = [0.0] * h
        for j in range(k):
            e = int(idx[mi, j])
            hid = []
            for r in range(f):
                g = sum(float(x[mi, c]) * wval(gus[e], r, c) for c in range(h))
                u = sum(float(x[mi, c]) * wval(gus[e], f + r, c) for c in range(h))
                hid.append(g / (1.0 + math.exp(-g)) * u)
            for r in range(h):
                acc[r] += float(wts[mi, j]) * sum(hid[c] * wval(dns[e], r, c) for c in range(f))
        np.testing.assert_allclose(y[mi], acc, rtol=1e-11, atol=1e-11)


# ------------------------------------------- integer q8 x q8 path (quantized activations)


def check_act_quant_hand(o):
    """Hand-derived codes and scales (tests/golden/q8_act_hand.txt): ties to even,
    the clamp at 127, powers-of-two scales, an all-zero block."""
    x = np.array([c["x"] for c in ACT_CASES], dtype=np.float32)
    q, dx = o.quantize_act_q8_ref(x)
    for i, c in enumerate(ACT_CASES):
        assert q[i].tolist() == c["q"], c["name"]
        assert float(dx[i, 0]) == c["dx"], c["name"]


def check_act_quant_props(o):
    """Codes within [-127, 127], 127 reached in every non-zero block, |x - q*dx| <= dx/2
    up to float32 rounding, zero blocks exact, and invariance under scaling by 2^j."""
    x = wl.activations(40, 5, 512)
    x[1, 64:96] = 0.0                       # one all-zero block
    x[2, 0:32] *= 1e-30                     # a block of tiny values
    q, dx = o.quantize_act_q8_ref(x)
    qb = q.reshape(5, 16, 32).astype(np.int64)
    xb = x.reshape(5, 16, 32).astype(np.float64)
    assert np.abs(qb).max() <= 127
    nz = np.abs(xb).max(axis=2) > 0
    assert np.all(np.abs(qb).max(axis=2)[nz] == 127)
    assert np.all(dx[~nz] == 0) and np.all(qb[~nz] == 0)
    err = np.abs(xb - qb * dx.astype(np.float64)[:, :, None])
    assert np.all(err <= 0.5 * dx.astype(np.float64)[:, :, None] * (1 + 1e-5) + 1e-45)
    for j in (-3, 5):
        q2, dx2 = o.quantize_act_q8_ref(x * np.float32(2.0 ** j))
        assert np.array_equal(q2, q)
        assert np.array_equal(dx2, (dx * np.float32(2.0 ** j)).astype(np.float32))


def check_q8act_linear(o):
    """The integer block-dot form equals dequantize-then-matmul of the quantized
    activations; lossless activations (x = q0 * 2^-3 with 127 in every block) give
    the plain linear; Fraction brute force on a tiny case."""
    n, k, m = 6, 256, 3
    wb, qw, dw = wl.q8_weight(41, n, k)
    x = wl.activations(42, m, k)
    y = o.q8_linear_q8act_ref(wb, n, k, x)
    qx, dx = o.quantize_act_q8_ref(x)
    xdq = (qx.reshape(m, k // 32, 32).astype(np.float64) * dx.astype(np.float64)[:, :, None]).reshape(m, k)
    np.testing.assert_allclose(y, o.q8_linear_ref(wb, n, k, xdq), rtol=1e-12, atol=1e-12)
    rng = np.random.default_rng(43)
    q0 = rng.integers(-127, 128, size=(m, k // 32, 32))
    q0[:, :, 7] = 127
    xl = (q0 * 2.0 ** -3).reshape(m, k).astype(np.float32)
    np.testing.assert_allclose(o.q8_linear_q8act_ref(wb, n, k, xl), o.q8_linear_ref(wb, n, k, xl),
                               rtol=1e-12, atol=1e-12)
    # arbitrary codes (the full int8 range, -128 included) against dequantize-then-matmul
    qa = rng.integers(-128, 128, size=(m, k)).astype(np.int8)
    da = (rng.random((m, k // 32)) * 0.01).astype(np.float32)
    xa = (qa.reshape(m, k // 32, 32).astype(np.float64) * da.astype(np.float64)[:, :, None]).reshape(m, k)
    np.testing.assert_allclose(o.q8_linear_codes_ref(wb, n, k, qa, da), o.q8_linear_ref(wb, n, k, xa),
                               rtol=1e-12, atol=1e-12)
    # brute force: n = 2, k = 64, m = 1, every product written out in rationals
    wb2, qw2, dw2 = wl.q8_weight(44, 2, 64)
    x2 = wl.activations(45, 1, 64)
    y2 = o.q8_linear_q8act_ref(wb2, 2, 64, x2)
    qx2, dx2 = o.quantize_act_q8_ref(x2)
    for ni in range(2):
        exact = Fraction(0)
        for kk in range(64):
            b = kk // 32
            exact += (half_bits_to_fraction(int(dw2.view(np.uint16)[ni, b])) * int(qw2[ni, kk])
                      * Fraction(float(dx2[0, b])) * int(qx2[0, kk]))
        assert abs(y2[0, ni] - float(exact)) <= 1e-12 * max(1.0, abs(float(exact)))


def check_q8act_fused(o):
    """The fused q8act SwiGLU is SiLU of the gate half times the up half."""
    f, k, m = 4, 256, 2
    wb, _, _ = wl.q8_weight(46, 2 * f, k)
    x = wl.activations(47, m, k)
    h = o.fused_gate_up_silu_q8act_ref(wb, f, k, x)
    y = o.q8_linear_q8act_ref(wb, 2 * f, k, x)
    np.testing.assert_allclose(h, scipy.special.expit(y[:, :f]) * y[:, :f] * y[:, f:], rtol=1e-12, atol=1e-15)


# ----------------------------------------------------- adaptive expert top-p routing


def _logit_router(logits):
    """x = logits, W_r = identity: the router's logits are exactly the given values."""
    logits = np.asarray(logits, dtype=np.float64)
    return logits, np.eye(logits.shape[1])


def check_top_p_exact_boundaries(o):
    """Equal logits give exact probabilities 1/E: the cut at c_{j-1} < top_p is checked
    exactly at the boundaries, and the cumulative is over the chosen k, not all E."""
    x, wr = _logit_router(np.zeros((1, 8)))
    for top_p, kept in ((0.25, 1), (0.26, 2), (0.5, 2), (0.51, 3), (0.75, 3), (0.76, 4), (1.0, 4)):
        idx, w = o.route_topk_p_ref(x, wr, 4, True, top_p)
        assert idx[0].tolist() == [0, 1, 2, 3][:kept] + [-1] * (4 - kept), (top_p, idx)
        np.testing.assert_allclose(w[0, :kept], 1.0 / kept, rtol=0, atol=1e-15)
        assert np.all(w[0, kept:] == 0)
    idx, w = o.route_topk_p_ref(x, wr, 4, False, 0.5)
    np.testing.assert_allclose(w[0], [0.125, 0.125, 0, 0], rtol=0, atol=1e-15)


def check_top_p_hand_and_identity(o):
    """Hand case p = (1/2, 1/4, 1/8, 1/8); top_p = 1 is plain top-k routing."""
    x, wr = _logit_router(np.log([[0.125, 0.5, 0.125, 0.25]]))
    for top_p, kept, wexp in ((0.4, 1, [1.0]), (0.6, 2, [2 / 3, 1 / 3]), (0.8, 3, [4 / 7, 2 / 7, 1 / 7]),
                              (0.9, 4, [0.5, 0.25, 0.125, 0.125])):
        idx, w = o.route_topk_p_ref(x, wr, 4, True, top_p)
        assert idx[0].tolist() == [1, 3, 0, 2][:kept] + [-1] * (4 - kept), (top_p, idx)
        np.testing.assert_allclose(w[0, :kept], wexp, rtol=1e-12)
    xr = wl.activations(71, 9, 256)
    w_r = wl.router_weight(72, 16, 256, std=0.1)
    for k in (1, 3, 8):
        for norm in (True, False):
            i1, w1 = o.route_topk_p_ref(xr, w_r, k, norm, 1.0)
            i0, w0 = o.route_topk_ref(xr, w_r, k, norm)
            assert np.array_equal(i1, i0)
            np.testing.assert_allclose(w1, w0, rtol=1e-14)


def check_top_p_properties(o):
    """Kept slots are a prefix, their count is 1 + #{j < k-1 : c_j < top_p} and grows
    with top_p; normalized kept weights sum to 1; the mixture of a top-p routing equals
    the mixture over the kept slots only."""
    xr = wl.activations(73, 12, 256)
    w_r = wl.router_weight(74, 32, 256, std=0.15)
    k = 6
    p_all = o.softmax_ref(o.router_logits_ref(xr, w_r))
    prev = None
    for top_p in (0.05, 0.3, 0.5, 0.7, 0.9, 0.99):
        idx, w = o.route_topk_p_ref(xr, w_r, k, True, top_p)
        kept = (idx >= 0).sum(axis=1)
        for m in range(12):
            assert np.all(idx[m, :kept[m]] >= 0) and np.all(idx[m, kept[m]:] == -1)
            chosen = np.sort(p_all[m])[::-1][:k]
            c = np.cumsum(chosen) / chosen.sum()
            assert kept[m] == 1 + int(np.sum(c[:k - 1] < top_p)), (m, top_p)
            assert abs(w[m, :kept[m]].sum() - 1.0) < 1e-12
        if prev is not None:
            assert np.all(kept >= prev)
        prev = kept
    # mixture: dropped slots contribute nothing
    e_n, hd, ff = 4, 256, 256
    gu = np.concatenate([wl.q8_weight(80 + e, 2 * ff, hd)[0] for e in range(e_n)])
    dn = np.concatenate([wl.q8_weight(90 + e, hd, ff)[0] for e in range(e_n)])
    xm = wl.activations(75, 2, hd)
    idx = np.array([[2, 0, -1], [1, -1, -1]], dtype=np.int32)
    wts = np.array([[0.75, 0.25, 0.0], [1.0, 0.0, 0.0]])
    y = o.moe_mixture_ref(gu, dn, e_n, ff, hd, xm, idx, wts)
    y0 = o.moe_mixture_ref(gu, dn, e_n, ff, hd, xm[:1], idx[:1, :2], wts[:1, :2])
    y1 = o.moe_mixture_ref(gu, dn, e_n, ff, hd, xm[1:], idx[1:, :1], wts[1:, :1])
    np.testing.assert_allclose(y, np.concatenate([y0, y1]), rtol=1e-14)


# ------------------------------------------------------------------------- Q4_0


def check_q4_0_hand(o):
    """Hand-derived blocks (tests/golden/q4_0_hand.txt): nibble order, the -8 offset, the
    sign and size of d; and a linear over those blocks against the hand weights."""
    for c in Q4_CASES:
        w = o.dequantize_q4_0(c["bytes"], 1, 32)
        assert w[0].tolist() == c["w"], c["name"]
    raw = b"".join(c["bytes"] for c in Q4_CASES)       # 4 rows of one block each
    x = wl.activations(91, 3, 32)
    wh = np.array([c["w"] for c in Q4_CASES])
    np.testing.assert_allclose(o.q4_0_linear_ref(raw, len(Q4_CASES), 32, x), x.astype(np.float64) @ wh.T,
                               rtol=1e-13)


def check_q4_0_properties(o):
    """Linearity in d, zero d gives zero, nibble 8 everywhere gives zero, Fraction brute
    force on a small case, and the fused split."""
    n, k = 5, 256
    wb, q, d = wl.q4_0_weight(92, n, k)
    x = wl.activations(93, 2, k)
    y = o.q4_0_linear_ref(wb, n, k, x)
    y2 = o.q4_0_linear_ref(wl.pack_q4_0(q, (d.astype(np.float32) * 2).astype(np.float16)), n, k, x)
    np.testing.assert_allclose(y2, 2 * y, rtol=1e-13)
    assert np.all(o.q4_0_linear_ref(wl.pack_q4_0(q, np.zeros_like(d)), n, k, x) == 0)
    assert np.all(o.q4_0_linear_ref(wl.pack_q4_0(np.full_like(q, 8), d), n, k, x) == 0)
    # brute force: one row, one block pair, every product in rationals
    wb1, q1, d1 = wl.q4_0_weight(94, 1, 64)
    x1 = wl.activations(95, 1, 64)
    exact = Fraction(0)
    for kk in range(64):
        dd = half_bits_to_fraction(int(d1.view(np.uint16)[0, kk // 32]))
        exact += dd * (int(q1[0, kk]) - 8) * Fraction(float(x1[0, kk]))
    assert abs(o.q4_0_linear_ref(wb1, 1, 64, x1)[0, 0] - float(exact)) <= 1e-12 * max(1.0, abs(float(exact)))
    f = 3
    wg, _, _ = wl.q4_0_weight(96, 2 * f, k)
    h = o.fused_gate_up_silu_q4_0_ref(wg, f, k, x)
    yy = o.q4_0_linear_ref(wg, 2 * f, k, x)
    np.testing.assert_allclose(h, scipy.special.expit(yy[:, :f]) * yy[:, :f] * yy[:, f:], rtol=1e-12, atol=1e-15)


# ------------------------------------------------------------------- Q4_K, Q6_K


def check_k_quant_hand(o):
    """Hand-derived super-blocks (tests/golden/k_quants_hand.txt): the packing of the 6-bit
    scales and mins, nibble order, the Q6_K bit-pair and index map, the -32 offset, scale
    groups; and a linear over the Q4_K blocks and one over the Q6_K blocks against the hand
    weights."""
    for fmt, deq, lin in (("q4_k", o.dequantize_q4_k, o.q4_k_linear_ref), ("q6_k", o.dequantize_q6_k,
                                                                          o.q6_k_linear_ref),
                          ("q5_k", o.dequantize_q5_k, o.q5_k_linear_ref)):
        cases = [c for c in KQ_CASES if c["format"] == fmt]
        for c in cases:
            w = deq(c["bytes"], 1, 256)
            assert w[0].tolist() == c["w"], c["name"]
        raw = b"".join(c["bytes"] for c in cases)
        x = wl.activations(97, 2, 256)
        wh = np.array([c["w"] for c in cases])
        np.testing.assert_allclose(lin(raw, len(cases), 256, x), x.astype(np.float64) @ wh.T, rtol=1e-13)


def check_k_quant_properties(o):
    """Fields drawn by the generator, combined by the format's formula in rationals (one
    super-block row, brute force), agree with the oracle's parse of the packed bytes;
    linearity in d (and dmin); zero quants; the fused split."""
    n, k = 3, 512
    wb, q, sc, mn, d, dmin = wl.q4_k_weight(98, n, k)
    x = wl.activations(99, 2, k)
    y = o.q4_k_linear_ref(wb, n, k, x)
    row, xr = 1, x[1]
    exact = Fraction(0)
    for i in range(k):
        b, j = i // 256, (i % 256) // 32
        dd = half_bits_to_fraction(int(d.view(np.uint16)[row, b]))
        dm = half_bits_to_fraction(int(dmin.view(np.uint16)[row, b]))
        exact += (dd * int(sc[row, b, j]) * int(q[row, i]) - dm * int(mn[row, b, j])) * Fraction(float(xr[i]))
    assert abs(y[1, row] - float(exact)) <= 1e-12 * max(1.0, abs(float(exact)))
    two = lambda a: (a.astype(np.float32) * 2).astype(np.float16)
    np.testing.assert_allclose(o.q4_k_linear_ref(wl.pack_q4_k(q, sc, mn, two(d), two(dmin)), n, k, x), 2 * y,
                               rtol=1e-13)
    z = o.q4_k_linear_ref(wl.pack_q4_k(np.zeros_like(q), sc, mn, d, np.zeros_like(dmin)), n, k, x)
    assert np.all(z == 0)
    wb6, q6, s6, d6 = wl.q6_k_weight(100, n, k)
    y6 = o.q6_k_linear_ref(wb6, n, k, x)
    exact = Fraction(0)
    for i in range(k):
        b = i // 256
        dd = half_bits_to_fraction(int(d6.view(np.uint16)[row, b]))
        exact += dd * int(s6[row, b, (i % 256) // 16]) * (int(q6[row, i]) - 32) * Fraction(float(xr[i]))
    assert abs(y6[1, row] - float(exact)) <= 1e-12 * max(1.0, abs(float(exact)))
    np.testing.assert_allclose(o.q6_k_linear_ref(wl.pack_q6_k(q6, s6, two(d6)), n, k, x), 2 * y6, rtol=1e-13)
    assert np.all(o.q6_k_linear_ref(wl.pack_q6_k(np.full_like(q6, 32), s6, d6), n, k, x) == 0)
    # Q5_K: rational brute force from the generator's fields; linearity in d and dmin
    wb5, q5, sc5, mn5, d5, dmin5 = wl.q5_k_weight(102, n, k)
    y5 = o.q5_k_linear_ref(wb5, n, k, x)
    exact = Fraction(0)
    for i in range(k):
        b, j = i // 256, (i % 256) // 32
        dd = half_bits_to_fraction(int(d5.view(np.uint16)[row, b]))
        dm = half_bits_to_fraction(int(dmin5.view(np.uint16)[row, b]))
        exact += (dd * int(sc5[row, b, j]) * int(q5[row, i]) - dm * int(mn5[row, b, j])) * Fraction(float(xr[i]))
    assert abs(y5[1, row] - float(exact)) <= 1e-12 * max(1.0, abs(float(exact)))
    np.testing.assert_allclose(o.q5_k_linear_ref(wl.pack_q5_k(q5, sc5, mn5, two(d5), two(dmin5)), n, k, x), 2 * y5,
                               rtol=1e-13)
    # Q5_K against Q4_K (pinned on its own above): with every top bit clear a Q5_K
    # super-block is the Q4_K one with the same fields; with every top bit set each weight
    # gains 16 * d * sc of its sub-block
    low = q5 & 15
    w4 = o.dequantize_q4_k(wl.pack_q4_k(low, sc5, mn5, d5, dmin5), n, k)
    assert np.array_equal(o.dequantize_q5_k(wl.pack_q5_k(low, sc5, mn5, d5, dmin5), n, k), w4)
    gain = 16 * np.repeat(d5.astype(np.float64)[:, :, None] * sc5.astype(np.float64), 32, axis=2).reshape(n, k)
    assert np.array_equal(o.dequantize_q5_k(wl.pack_q5_k(low | 16, sc5, mn5, d5, dmin5), n, k), w4 + gain)
    f = 3
    for lin, fused, gen in ((o.q4_k_linear_ref, o.fused_gate_up_silu_q4_k_ref, wl.q4_k_weight),
                            (o.q5_k_linear_ref, o.fused_gate_up_silu_q5_k_ref, wl.q5_k_weight),
                            (o.q6_k_linear_ref, o.fused_gate_up_silu_q6_k_ref, wl.q6_k_weight)):
        wg = gen(101, 2 * f, k)[0]
        h = fused(wg, f, k, x)
        yy = lin(wg, 2 * f, k, x)
        np.testing.assert_allclose(h, scipy.special.expit(yy[:, :f]) * yy[:, :f] * yy[:, f:], rtol=1e-12,
                                   atol=1e-15)


ALL_CHECKS = [
    check_hand_linear, check_hand_fused, check_hand_route, check_bruteforce_linear,
    check_dequant_exact, check_linearity, check_zero_scale, check_one_hot, check_silu,
    check_fused_split, check_route_invariants, check_moe, check_moe_bruteforce,
    check_act_quant_hand, check_act_quant_props, check_q8act_linear, check_q8act_fused,
    check_top_p_exact_boundaries, check_top_p_hand_and_identity, check_top_p_properties,
    check_q4_0_hand, check_q4_0_properties, check_k_quant_hand, check_k_quant_properties,
]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(O)


def test_bf16_rounding_diag():
    # bfloat16 keeps 7 fraction bits: 1 + 2^-8 is a tie (to even: 1), 1 + 3*2^-8 is a
    # tie between 1 + 2^-7 (odd) and 1 + 2^-6 (even), 1 + 2^-7 is representable
    vals = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2.0 ** 100 * (1 + 2 ** -8), 1 + 2 ** -7])
    want = np.array([1.0, 1.0, 1 + 2 ** -6, -1.0, 2.0 ** 100, 1 + 2 ** -7])
    got = O.bf16_round_ref(vals)
    assert np.array_equal(got, want)


def test_error_measures():
    ref = np.array([[3.0, 4.0], [0.0, 0.0]])
    assert O.rel_err_row_norm(ref, ref) == 0.0
    assert O.rel_err_row_norm(ref + np.array([[0.5, 0.0], [0.0, 0.0]]), ref) == pytest.approx(0.1)
    assert O.rel_err_row_max(ref + np.array([[0.5, 0.0], [0.0, 0.0]]), ref) == pytest.approx(0.125)
    assert O.rel_err_row_norm(ref + np.array([[0.0, 0.0], [0.0, 1e-3]]), ref) == math.inf


def test_parse_rejects_bad_sizes():
    with pytest.raises(ValueError):
        O.parse_q8_0(b"\x00" * 33, 1, 32)
    with pytest.raises(ValueError):
        O.q8_0_row_bytes(48)
