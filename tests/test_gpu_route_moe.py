"""GPU parity of moe_route_topk and q8_moe_grouped_linear against the CPU oracle.

Router indices must match exactly wherever the choice is unique at float32 precision:
the oracle's float64 logits decide, and positions whose logit gap is within the rounding
bound of the two float32 logits (see logit_error_bound) are checked for validity instead
(every chosen expert within that bound of the true order).  Exactly representable logits
(small integers) must match bit for bit, ties included.  For the Qwen3-30B-A3B layer's
own seed every index must equal the oracle's.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import TOL, assert_close, moe_mixture_grouped_ref, say, to_dev, torch_dev

pytestmark = pytest.mark.gpu



def logit_error_bound(x, wr):
    """Bound on |float32 logit - exact logit| per (token, expert): gamma_d * sum_i |x_i w_i|
    with gamma_d = d*u / (1 - d*u), u = 2^-24, the standard bound for a float32 sum in which
    every term passes through at most d roundings.  The router sums each lane's h/64 inputs
    in one chain and then the 64 lane partials in a fixed tree of at most 7 levels (four
    within 16-lane rows, then three across the rows), so d = h/64 + 8 covers the product's
    own rounding as well."""
    h = x.shape[1]
    d = h // 64 + 8
    u = 2.0 ** -24
    gamma = d * u / (1 - d * u)
    return gamma * (np.abs(x.astype(np.float64)) @ np.abs(wr.astype(np.float64)).T)


@pytest.fixture(scope="module")
def q8():
    torch, dev = torch_dev()
    import block_quantized_weight_linear_amd as q8mod
    return q8mod, torch, dev


def check_routing(idx_gpu, w_gpu, x, wr, k, normalize):
    """Returns the number of tokens whose choice was ambiguous at float32 precision."""
    ridx, rw = oracle.route_topk_ref(x, wr, k, normalize)
    logits = oracle.router_logits_ref(x, wr)
    bound = logit_error_bound(x, wr)
    ambiguous = 0
    for t in range(x.shape[0]):
        order = np.argsort(-logits[t], kind="stable")
        srt = logits[t, order]
        # positions j and j+1 are ordered for certain when their gap exceeds both bounds
        sep = (srt[:-1] - srt[1:]) > (bound[t, order[:-1]] + bound[t, order[1:]])
        unique = all((j == 0 or sep[j - 1]) and (j >= len(sep) or sep[j]) for j in range(k))
        if unique:
            assert idx_gpu[t].tolist() == ridx[t].tolist(), (t, idx_gpu[t], ridx[t])
            np.testing.assert_allclose(w_gpu[t], rw[t], rtol=TOL, atol=TOL * np.abs(rw[t]).max())
        else:
            ambiguous += 1
            chosen = idx_gpu[t]
            assert len(set(chosen.tolist())) == k
            tol = 2 * bound[t].max()
            kth = srt[k - 1]
            assert np.all(logits[t, chosen] >= kth - tol), t
            assert np.all(np.diff(logits[t, chosen]) <= tol), t
    return ambiguous


def _pad_h(a, h=256):
    out = np.zeros((a.shape[0], h), np.float32)
    out[:, :a.shape[1]] = a
    return out


def test_hand_router_cases(q8):
    from golden_io import load_swiglu_router_cases
    lib, torch, dev = q8
    _, cases = load_swiglu_router_cases()
    for c in cases:
        x = _pad_h(np.array(c["x"], np.float32))
        wr = _pad_h(np.array(c["w_router"], np.float32))
        idx, w = lib.moe_route_topk(to_dev(x, dev), to_dev(wr, dev), c["k"], c["normalize"])
        assert idx.cpu().numpy().tolist() == c["idx"], c["name"]
        np.testing.assert_allclose(w.cpu().numpy(), np.array(c["w"]), rtol=1e-6, err_msg=c["name"])


def test_exact_logits_with_ties(q8):
    """Integer activations and router rows: float32 logits are exact, ties included."""
    lib, torch, dev = q8
    m, h, e = 64, 512, 40
    rng = np.random.default_rng(7)
    x = rng.integers(-1, 2, size=(m, h)).astype(np.float32)
    wr = rng.integers(-1, 2, size=(e, h)).astype(np.float32)
    wr[5] = wr[3]      # guaranteed ties
    wr[17] = wr[3]
    for k in (1, 4, 8, e):
        idx, w = lib.moe_route_topk(to_dev(x, dev), to_dev(wr, dev), k, True)
        ridx, rw = oracle.route_topk_ref(x, wr, k, True)
        assert np.array_equal(idx.cpu().numpy(), ridx), k
        np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("m,h,e,k,normalize", [(16, 2048, 128, 8, True), (16, 2048, 128, 8, False),
                                               (257, 1024, 64, 6, True), (3, 256, 256, 256, True),
                                               (1, 4096, 8, 2, True), (33, 768, 7, 1, True)])
def test_router_vs_oracle(q8, m, h, e, k, normalize):
    lib, torch, dev = q8
    x = wl.activations(81 + m, m, h)
    wr = wl.router_weight(82 + e, e, h)
    say(f"router m={m} h={h} e={e} k={k}")
    idx, w = lib.moe_route_topk(to_dev(x, dev), to_dev(wr, dev), k, normalize)
    amb = check_routing(idx.cpu().numpy(), w.cpu().numpy(), x, wr, k, normalize)
    say(f"router m={m}: {amb} ambiguous tokens")
    if k == e and normalize:
        p = oracle.softmax_ref(oracle.router_logits_ref(x, wr))
        got = np.zeros_like(p)
        np.put_along_axis(got, idx.cpu().numpy().astype(np.int64), w.cpu().numpy(), axis=1)
        assert_close(got, p, "k=E full softmax")


# ------------------------------------------------------------------------- MoE


def _experts(seed, e, f, h):
    gu = np.concatenate([wl.q8_weight(seed + i, 2 * f, h)[0] for i in range(e)])
    dn = np.concatenate([wl.q8_weight(seed + 1000 + i, h, f)[0] for i in range(e)])
    return gu, dn


@pytest.fixture(scope="module")
def a3b_layer():
    cfg = wl.QWEN3_30B_A3B_MOE
    gu, dn = _experts(cfg.seed * 10000, cfg.n_exp, cfg.ffn, cfg.hidden)
    x = wl.activations(cfg.seed + 1, cfg.tokens, cfg.hidden)
    wr = wl.router_weight(cfg.seed + 2, cfg.n_exp, cfg.hidden, cfg.router_std)
    return cfg, gu, dn, x, wr


def test_moe_layer_given_routing(q8, a3b_layer):
    lib, torch, dev = q8
    cfg, gu, dn, x, wr = a3b_layer
    ridx, rw = oracle.route_topk_ref(x, wr, cfg.k, True)
    say("moe 30b-a3b layer, oracle routing")
    y = lib.q8_moe_grouped_linear(to_dev(gu, dev), to_dev(dn, dev), cfg.n_exp, cfg.ffn, cfg.hidden, to_dev(x, dev),
                                  to_dev(ridx.astype(np.int32), dev), to_dev(rw.astype(np.float32), dev)).cpu().numpy()
    ref = oracle.moe_mixture_ref(gu, dn, cfg.n_exp, cfg.ffn, cfg.hidden, x, ridx, rw.astype(np.float32))
    assert_close(y, ref, "moe 30b-a3b layer (given routing)")


def test_moe_layer_end_to_end(q8, a3b_layer):
    """Device routing then the device mixture.  Where the routing choice is unique at
    float32 precision it equals the oracle's (checked in check_routing); the mixture is
    compared with the oracle's mixture for the experts the device chose, weighted by the
    oracle's float64 softmax renormalized over those experts."""
    lib, torch, dev = q8
    cfg, gu, dn, x, wr = a3b_layer
    xd = to_dev(x, dev)
    idx, w = lib.moe_route_topk(xd, to_dev(wr, dev), cfg.k, True)
    idx_h = idx.cpu().numpy()
    amb = check_routing(idx_h, w.cpu().numpy(), x, wr, cfg.k, True)
    # The layer's own seed: the chosen set is provably unique at float32 precision for every
    # token (the gap between the k-th and (k+1)-th logit exceeds the two rounding bounds),
    # and every index, order included, must equal the oracle's.
    ridx, _ = oracle.route_topk_ref(x, wr, cfg.k, True)
    logits = oracle.router_logits_ref(x, wr)
    bound = logit_error_bound(x, wr)
    margins = []
    for t in range(cfg.tokens):
        order = np.argsort(-logits[t], kind="stable")
        a, b = order[cfg.k - 1], order[cfg.k]
        margins.append((logits[t, a] - logits[t, b]) / (bound[t, a] + bound[t, b]))
    say(f"moe 30b-a3b layer: {amb} of {cfg.tokens} tokens with an order within the float32 bound; "
        f"smallest selection margin {min(margins):.1f}x the bound")
    assert min(margins) > 1.0, margins
    assert np.array_equal(idx_h, ridx), (idx_h, ridx)
    y = lib.q8_moe_grouped_linear(to_dev(gu, dev), to_dev(dn, dev), cfg.n_exp, cfg.ffn, cfg.hidden, xd, idx,
                                  w).cpu().numpy()
    p = oracle.softmax_ref(oracle.router_logits_ref(x, wr))
    w_ref = np.take_along_axis(p, idx_h.astype(np.int64), axis=1)
    w_ref = w_ref / w_ref.sum(axis=1, keepdims=True)
    ref = oracle.moe_mixture_ref(gu, dn, cfg.n_exp, cfg.ffn, cfg.hidden, x, idx_h, w_ref)
    assert_close(y, ref, "moe 30b-a3b layer (device routing)")
    y2 = lib.q8_moe_grouped_linear(to_dev(gu, dev), to_dev(dn, dev), cfg.n_exp, cfg.ffn, cfg.hidden, xd, idx,
                                   w).cpu().numpy()
    assert np.array_equal(y, y2)  # deterministic


MOE_PREFILL_TOL = 2e-2   # bf16 operands (x, d*q, and the hidden SiLU*up), float32 accumulation


# the mixture runs on the bf16 matrix-core tiles from this many routed pairs per expert
# on average (q8_moe_grouped_linear's documented switch point), else on the float32 passes
MATRIX_CORE_PAIRS_PER_EXPERT = 8


@pytest.mark.parametrize("m,e,k,f,h", [(1, 8, 2, 256, 512), (37, 16, 4, 512, 256), (64, 4, 2, 256, 1024),
                                       (5, 3, 3, 768, 2048), (200, 32, 8, 256, 256), (1000, 128, 6, 256, 256),
                                       (700, 256, 8, 256, 256), (100, 128, 8, 256, 512), (300, 256, 6, 256, 256),
                                       (20, 16, 6, 512, 256)])
def test_moe_shapes_vs_oracle(q8, m, e, k, f, h):
    """Float32 passes below 8 routed pairs per expert (several passes for experts with more
    than 4 tokens: 100 tokens x 8 slots over 128 experts, 300 x 6 over 256, 20 x 6 over
    16), bf16 tiles from there on, each at its tolerance."""
    lib, torch, dev = q8
    tol = MOE_PREFILL_TOL if m * k >= MATRIX_CORE_PAIRS_PER_EXPERT * e else TOL
    gu, dn = _experts(500 + e, e, f, h)
    x = wl.activations(90 + m, m, h)
    idx, w = wl.random_routing(91 + m, m, e, k)
    say(f"moe m={m} e={e} k={k} f={f} h={h}")
    y = lib.q8_moe_grouped_linear(to_dev(gu, dev), to_dev(dn, dev), e, f, h, to_dev(x, dev), to_dev(idx, dev),
                                  to_dev(w, dev)).cpu().numpy()
    assert_close(y, oracle.moe_mixture_ref(gu, dn, e, f, h, x, idx, w), f"moe m={m} e={e}", tol=tol)


def test_moe_k1_equals_dense_ffn_bitwise(q8):
    """k = 1 with weight 1: the mixture is the chosen expert's dense SwiGLU FFN, and the
    grouped kernels do the same per-row arithmetic as the dense calls."""
    lib, torch, dev = q8
    e, f, h, m = 6, 768, 2048, 9
    gu, dn = _experts(700, e, f, h)
    x = wl.activations(701, m, h)
    idx = np.array([[i % e] for i in range(m)], np.int32)
    w = np.ones((m, 1), np.float32)
    gud, dnd, xd = to_dev(gu, dev), to_dev(dn, dev), to_dev(x, dev)
    y = lib.q8_moe_grouped_linear(gud, dnd, e, f, h, xd, to_dev(idx, dev), to_dev(w, dev)).cpu().numpy()
    gu_b = (2 * f) * (h // 32) * 34
    dn_b = h * (f // 32) * 34
    for t in range(m):
        ex = int(idx[t, 0])
        hid = lib.q8_linear_fused_gate_up_silu(gud[ex * gu_b:(ex + 1) * gu_b], f, h, xd[t:t + 1].contiguous())
        out = lib.q8_linear(dnd[ex * dn_b:(ex + 1) * dn_b], h, f, hid).cpu().numpy()
        assert np.array_equal(y[t], out[0]), t


def test_moe_relabel_and_duplicates(q8):
    lib, torch, dev = q8
    e, f, h, m, k = 5, 256, 512, 11, 3
    gu, dn = _experts(800, e, f, h)
    x = wl.activations(801, m, h)
    idx, w = wl.random_routing(802, m, e, k)
    xd = to_dev(x, dev)
    y = lib.q8_moe_grouped_linear(to_dev(gu, dev), to_dev(dn, dev), e, f, h, xd, to_dev(idx, dev),
                                  to_dev(w, dev)).cpu().numpy()
    perm = np.array([3, 0, 4, 1, 2])           # new expert i holds old expert perm[i]
    gu_b = (2 * f) * (h // 32) * 34
    dn_b = h * (f // 32) * 34
    gu_p = np.concatenate([gu[p * gu_b:(p + 1) * gu_b] for p in perm])
    dn_p = np.concatenate([dn[p * dn_b:(p + 1) * dn_b] for p in perm])
    inv = np.argsort(perm)
    idx_p = inv[idx].astype(np.int32)
    yp = lib.q8_moe_grouped_linear(to_dev(gu_p, dev), to_dev(dn_p, dev), e, f, h, xd, to_dev(idx_p, dev),
                                   to_dev(w, dev)).cpu().numpy()
    assert np.array_equal(y, yp)
    # the same expert twice in one token's slots, and an out-of-range id that is skipped
    idx2 = idx.copy()
    idx2[:, 1] = idx2[:, 0]
    idx2[0, 2] = e + 7
    y2 = lib.q8_moe_grouped_linear(to_dev(gu, dev), to_dev(dn, dev), e, f, h, xd, to_dev(idx2, dev),
                                   to_dev(w, dev)).cpu().numpy()
    ref_idx = idx2.copy()
    ref_w = w.copy()
    ref_idx[0, 2] = 0
    ref_w[0, 2] = 0.0
    assert_close(y2, oracle.moe_mixture_ref(gu, dn, e, f, h, x, ref_idx, ref_w), "duplicates + skipped id")


# ------------------------------------------------------ adaptive expert top-p routing


def check_top_p(idx_gpu, w_gpu, x, wr, k, normalize, top_p, eps=1e-5):
    """Kept slots are a prefix with expert -1 / weight 0 after it; the kept count equals
    the oracle's wherever no cumulative share c_j lies within eps of top_p (else it lies in
    the band the float32 rounding allows); kept experts are the top-k's leading ones."""
    ridx, rw = oracle.route_topk_p_ref(x, wr, k, normalize, top_p)
    tidx, _ = oracle.route_topk_ref(x, wr, k, normalize)
    p = oracle.softmax_ref(oracle.router_logits_ref(x, wr))
    for t in range(x.shape[0]):
        kept = int((idx_gpu[t] >= 0).sum())
        assert kept >= 1 and np.all(idx_gpu[t, :kept] >= 0) and np.all(idx_gpu[t, kept:] == -1), t
        assert np.all(w_gpu[t, kept:] == 0), t
        chosen = p[t, tidx[t]]
        c = np.cumsum(chosen) / chosen.sum()
        lo = 1 + int(np.sum(c[:k - 1] < top_p - eps))
        hi = 1 + int(np.sum(c[:k - 1] < top_p + eps))
        if top_p >= 1.0:
            lo = hi = k
        assert lo <= kept <= hi, (t, kept, lo, hi)
        if lo == hi:
            rk = int((ridx[t] >= 0).sum())
            assert kept == rk
        if normalize:
            assert abs(float(w_gpu[t, :kept].sum()) - 1.0) < 1e-5, t
        else:
            np.testing.assert_allclose(w_gpu[t, :kept], chosen[:kept], rtol=TOL)


def test_top_p_one_is_plain_topk(q8):
    lib, torch, dev = q8
    x = wl.activations(201, 33, 2048)
    wr = wl.router_weight(202, 128, 2048)
    xd, wd = to_dev(x, dev), to_dev(wr, dev)
    for k, norm in ((8, True), (8, False), (1, True), (128, True)):
        i0, w0 = lib.moe_route_topk(xd, wd, k, norm)
        i1, w1 = lib.moe_route_topk(xd, wd, k, norm, top_p=1.0)
        assert torch.equal(i0, i1) and torch.equal(w0, w1), k


def test_top_p_exact_boundaries(q8):
    """Zero activations: every logit is 0 and every probability exactly 1/E (E a power of
    two), so the cut is decided exactly, at the boundaries included."""
    lib, torch, dev = q8
    x = np.zeros((3, 256), np.float32)
    wr = wl.router_weight(203, 8, 256)
    for top_p, kept in ((0.25, 1), (0.26, 2), (0.5, 2), (0.51, 3), (0.75, 3), (0.76, 4), (1.0, 4)):
        idx, w = lib.moe_route_topk(to_dev(x, dev), to_dev(wr, dev), 4, True, top_p=top_p)
        ridx, rw = oracle.route_topk_p_ref(x, wr, 4, True, top_p)
        assert np.array_equal(idx.cpu().numpy(), ridx), (top_p, idx)
        assert int((ridx[0] >= 0).sum()) == kept
        np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=1e-6)
    idx, w = lib.moe_route_topk(to_dev(x, dev), to_dev(wr, dev), 4, False, top_p=0.5)
    assert np.array_equal(w.cpu().numpy()[0], np.array([0.125, 0.125, 0, 0], np.float32))


@pytest.mark.parametrize("top_p", [0.05, 0.3, 0.6, 0.9, 0.97])
@pytest.mark.parametrize("normalize", [True, False])
def test_top_p_vs_oracle(q8, top_p, normalize):
    lib, torch, dev = q8
    m, h, e, k = 64, 2048, 128, 8
    x = wl.activations(204, m, h)
    wr = wl.router_weight(205, e, h, std=0.05)   # spread logits: cuts at varied depths
    say(f"top-p router top_p={top_p} normalize={normalize}")
    idx, w = lib.moe_route_topk(to_dev(x, dev), to_dev(wr, dev), k, normalize, top_p=top_p)
    idx, w = idx.cpu().numpy(), w.cpu().numpy()
    check_top_p(idx, w, x, wr, k, normalize, top_p)
    # the kept experts are the leading ones of the device's plain top-k
    i0, _ = lib.moe_route_topk(to_dev(x, dev), to_dev(wr, dev), k, normalize)
    i0 = i0.cpu().numpy()
    kept = (idx >= 0)
    assert np.array_equal(idx[kept], i0[kept])
    say(f"top-p {top_p}: mean experts kept {kept.sum(axis=1).mean():.2f} of {k}")


def test_top_p_mixture(q8):
    """The grouped mixture on a top-p routing (dropped slots: expert -1) matches the oracle
    mixture on the same routing (float32 passes: 4 slots per expert; the bf16 tiles with a
    top-p routing are covered by the A3B prefill test)."""
    lib, torch, dev = q8
    m, e, f, h, k = 16, 32, 256, 512, 8
    assert m * k < MATRIX_CORE_PAIRS_PER_EXPERT * e
    gu, dn = _experts(300, e, f, h)
    x = wl.activations(206, m, h)
    wr = wl.router_weight(207, e, h, std=0.1)
    xd = to_dev(x, dev)
    idx, w = lib.moe_route_topk(xd, to_dev(wr, dev), k, True, top_p=0.6)
    assert int((idx < 0).sum()) > 0      # some slots were dropped
    y = lib.q8_moe_grouped_linear(to_dev(gu, dev), to_dev(dn, dev), e, f, h, xd, idx, w).cpu().numpy()
    ref = oracle.moe_mixture_ref(gu, dn, e, f, h, x, idx.cpu().numpy(), w.cpu().numpy().astype(np.float64))
    assert_close(y, ref, "top-p mixture")


# ------------------------------------------------------------- two-pass router


@pytest.mark.parametrize("m,h,e,k", [(16, 2048, 128, 8), (1, 4096, 8, 2), (257, 1024, 64, 6), (3, 256, 256, 256),
                                     (5, 6144, 7, 1), (33, 768, 130, 9), (2048, 2048, 128, 8), (1000, 768, 130, 9),
                                     (1000, 512, 7, 2), (384, 256, 256, 8), (383, 256, 256, 8)])
def test_two_pass_router_bit_identical(q8, m, h, e, k):
    """moe_route_topk_ws (logits over many CUs, then selection) equals the one-pass router
    bit for bit, with and without the top-p cut, and stays within the oracle's checks.
    From 384 tokens the logits run in 16-token x 32-expert tiles (ragged token and expert
    tiles here: 1000 tokens, 130 and 7 experts)."""
    lib, torch, dev = q8
    x = wl.activations(401 + m, m, h)
    wr = wl.router_weight(402 + e, e, h, std=0.05)
    xd, wd = to_dev(x, dev), to_dev(wr, dev)
    say(f"two-pass router m={m} h={h} e={e} k={k}")
    ws = torch.full((lib.moe_route_workspace_bytes(m, e),), 255, dtype=torch.uint8, device=dev)
    for norm in (True, False):
        i1, w1 = lib.moe_route_topk(xd, wd, k, norm)
        i2, w2 = lib.moe_route_topk(xd, wd, k, norm, workspace=ws)
        assert torch.equal(i1, i2) and torch.equal(w1, w2), norm
        for top_p in (0.3, 0.8):
            i1, w1 = lib.moe_route_topk(xd, wd, k, norm, top_p=top_p)
            i2, w2 = lib.moe_route_topk(xd, wd, k, norm, top_p=top_p, workspace=ws)
            assert torch.equal(i1, i2) and torch.equal(w1, w2), (norm, top_p)
    i2, w2 = lib.moe_route_topk(xd, wd, k, True, workspace=True)
    check_routing(i2.cpu().numpy(), w2.cpu().numpy(), x, wr, k, True)


def test_moe_graph_replay_matches_eager(q8):
    """Two-pass routing (with a top-p cut) and the grouped mixture captured in one HIP
    graph: every replay, with eager work and synchronizations in between, gives the eager
    result bit for bit (the route plan clears its counters with kernels, no memsets)."""
    lib, torch, dev = q8
    m, e, f, h, k = 16, 32, 256, 512, 4
    gu, dn = _experts(500, e, f, h)
    gud, dnd = to_dev(gu, dev), to_dev(dn, dev)
    xd = to_dev(wl.activations(501, m, h), dev)
    wrd = to_dev(wl.router_weight(502, e, h, std=0.1), dev)
    idx = torch.empty((m, k), dtype=torch.int32, device=dev)
    wts = torch.empty((m, k), device=dev)
    y = torch.empty((m, h), device=dev)
    ws_r = torch.empty(lib.moe_route_workspace_bytes(m, e), dtype=torch.uint8, device=dev)
    ws_m = torch.empty(lib.q8_moe_workspace_bytes(m, k, e, f, h), dtype=torch.uint8, device=dev)

    def step():
        lib.moe_route_topk(xd, wrd, k, True, idx_out=idx, w_out=wts, top_p=0.7, workspace=ws_r)
        lib.q8_moe_grouped_linear(gud, dnd, e, f, h, xd, idx, wts, out=y, workspace=ws_m)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (idx, wts, y)]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            step()
    for rep in range(4):
        y.fill_(float("nan"))
        idx.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((idx, wts, y), ref):
            assert torch.equal(got, want), rep
        step()
        torch.cuda.synchronize()


# ------------------------------------------- MoE prefill: expert-grouped matrix-core tiles



@pytest.mark.parametrize("m,e,k,f,h", [(300, 8, 2, 256, 512), (700, 16, 4, 512, 1024), (129, 2, 1, 768, 256),
                                       (520, 4, 3, 256, 2048)])
def test_moe_prefill_vs_oracle(q8, m, e, k, f, h):
    """At least 8 routed pairs per expert: the expert-grouped bf16 tiles run (ragged last
    tile of every expert, experts with fewer rows than a tile)."""
    lib, torch, dev = q8
    assert m * k >= MATRIX_CORE_PAIRS_PER_EXPERT * e
    gu, dn = _experts(900 + e, e, f, h)
    x = wl.activations(901 + m, m, h)
    idx, w = wl.random_routing(902 + m, m, e, k)
    say(f"moe prefill m={m} e={e} k={k} f={f} h={h}")
    y = lib.q8_moe_grouped_linear(to_dev(gu, dev), to_dev(dn, dev), e, f, h, to_dev(x, dev), to_dev(idx, dev),
                                  to_dev(w, dev)).cpu().numpy()
    assert_close(y, oracle.moe_mixture_ref(gu, dn, e, f, h, x, idx, w), f"moe prefill m={m} e={e}",
                 tol=MOE_PREFILL_TOL)
    y2 = lib.q8_moe_grouped_linear(to_dev(gu, dev), to_dev(dn, dev), e, f, h, to_dev(x, dev), to_dev(idx, dev),
                                   to_dev(w, dev)).cpu().numpy()
    assert np.array_equal(y, y2)  # deterministic


def test_moe_prefill_a3b_full(q8):
    """Qwen3-30B-A3B layer at 1024 tokens (8192 routed pairs, 64 per expert on average):
    device routing, then the grouped tiles; every output of all 1024 tokens against the
    oracle's mixture (its calls grouped by expert); dropped slots of a top-p routing are
    skipped on this path too."""
    lib, torch, dev = q8
    cfg = wl.QWEN3_30B_A3B_MOE
    e, f, h, k, m = cfg.n_exp, cfg.ffn, cfg.hidden, cfg.k, 1024
    gu, dn = _experts(950, e, f, h)
    x = wl.activations(951, m, h)
    wr = wl.router_weight(952, e, h, cfg.router_std)
    gud, dnd, xd = to_dev(gu, dev), to_dev(dn, dev), to_dev(x, dev)
    for top_p in (None, 0.8):
        say(f"moe prefill a3b m={m} top_p={top_p}")
        idx, w = lib.moe_route_topk(xd, to_dev(wr, dev), k, True, top_p=top_p, workspace=True)
        y = lib.q8_moe_grouped_linear(gud, dnd, e, f, h, xd, idx, w).cpu().numpy()
        idx_h, w_h = idx.cpu().numpy(), w.cpu().numpy().astype(np.float64)
        ref = moe_mixture_grouped_ref(gu, dn, e, f, h, x, idx_h, w_h)
        assert_close(y, ref, f"a3b prefill top_p={top_p} (all {m} tokens)", tol=MOE_PREFILL_TOL)
