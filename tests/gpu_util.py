"""Helpers shared by the GPU parity tests (device transfers, full-size oracle results in
row chunks, error measures)."""

from __future__ import annotations

import sys

import numpy as np
import pytest

TOL = 2e-3          # max relative error for float32 outputs (row-norm reading; also row-max)
Q8_BLOCK = 34


def torch_dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch, torch.device("cuda:0")


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def to_dev(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def row_slice(wbytes: np.ndarray, k: int, rows) -> np.ndarray:
    """Q8_0 bytes of the given rows (in order) of a matrix with row length k."""
    rb = (k // 32) * Q8_BLOCK
    w2 = wbytes.reshape(-1, rb)
    return np.ascontiguousarray(w2[np.asarray(rows)]).reshape(-1)


def sample_rows(n: int, count: int, seed: int = 0):
    """Sorted distinct rows: the first, the last, and `count` random ones."""
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(n, size=min(count, n), replace=False).tolist())
    pick.update({0, n - 1})
    return np.array(sorted(pick))


def assert_close(got, ref, what, tol=TOL):
    import oracle
    e1 = oracle.rel_err_row_norm(got, ref)
    e2 = oracle.rel_err_row_max(got, ref)
    say(f"{what}: rel err (row norm) {e1:.2e}, (row max) {e2:.2e}")
    assert e1 <= tol and e2 <= tol, (what, e1, e2)


def _n_rows(x) -> int:
    """Activation rows of x, or of the codes when x is a (codes, scales) pair."""
    return (x[0] if isinstance(x, tuple) else np.asarray(x)).shape[0]


def _row_range(wbytes: np.ndarray, k: int, r0: int, r1: int, block_bytes: float = Q8_BLOCK) -> np.ndarray:
    """Rows r0 .. r1-1 of a packed matrix; block_bytes is the bytes per 32 weights (210/8
    for Q6_K, whose 256-weight super-blocks are 210 bytes)."""
    rb = k * block_bytes / 32
    assert rb == int(rb), (k, block_bytes)
    rb = int(rb)
    return wbytes[r0 * rb:r1 * rb]


def linear_ref_full(wbytes, n: int, k: int, x, chunk: int = 2048, ref=None, block_bytes: int = Q8_BLOCK):
    """Every output of the oracle's linear (default oracle.q8_linear_ref), computed on row
    slices of the weight so host memory stays bounded at any matrix size.  ref(w, rows, k,
    x) is the oracle function to apply; the result is [m][n] float64."""
    import oracle
    ref = ref or oracle.q8_linear_ref
    out = np.empty((_n_rows(x), n), dtype=np.float64)
    for r0 in range(0, n, chunk):
        r1 = min(n, r0 + chunk)
        out[:, r0:r1] = ref(_row_range(wbytes, k, r0, r1, block_bytes), r1 - r0, k, x)
    return out


def fused_ref_full(wbytes, f: int, k: int, x, chunk: int = 2048, ref=None, block_bytes: int = Q8_BLOCK):
    """Every output of the oracle's fused gate_up (default oracle.fused_gate_up_silu_ref) on
    a [2f][k] matrix: each chunk of outputs is the oracle function on the matching gate
    rows followed by the matching up rows."""
    import oracle
    ref = ref or oracle.fused_gate_up_silu_ref
    out = np.empty((_n_rows(x), f), dtype=np.float64)
    for r0 in range(0, f, chunk):
        r1 = min(f, r0 + chunk)
        sub = np.concatenate([_row_range(wbytes, k, r0, r1, block_bytes),
                              _row_range(wbytes, k, f + r0, f + r1, block_bytes)])
        out[:, r0:r1] = ref(sub, r1 - r0, k, x)
    return out


def codes_ref(fn):
    """Adapts an oracle function of (w, rows, k, qx, dx) to the (w, rows, k, x) form used
    by linear_ref_full / fused_ref_full, with x = (qx, dx)."""
    return lambda w, rows, k, x: fn(w, rows, k, x[0], x[1])


def moe_mixture_grouped_ref(gu, dn, n_exp: int, f: int, h: int, x, idx, w):
    """The oracle's SwiGLU expert mixture with its calls grouped by expert: for each expert,
    oracle.fused_gate_up_silu_ref and oracle.q8_linear_ref run once on all the (token,
    slot) pairs routed to it; the per-pair outputs are then summed per token in slot order
    j = 0..k-1, as oracle.moe_mixture_ref does (equal to it up to float64 rounding; pinned
    against it on the CPU).  Slots with an expert id of -1 contribute nothing."""
    import oracle
    x64 = np.asarray(x, dtype=np.float64)
    idx = np.asarray(idx)
    w = np.asarray(w, dtype=np.float64)
    m, k = idx.shape
    gu_b = (2 * f) * (h // 32) * Q8_BLOCK
    dn_b = h * (f // 32) * Q8_BLOCK
    per_pair = np.zeros((m, k, h), dtype=np.float64)
    for e in range(n_exp):
        t, j = np.nonzero(idx == e)
        if t.size == 0:
            continue
        hid = oracle.fused_gate_up_silu_ref(gu[e * gu_b:(e + 1) * gu_b], f, h, x64[t])
        per_pair[t, j] = oracle.q8_linear_ref(dn[e * dn_b:(e + 1) * dn_b], h, f, hid)
    y = np.zeros((m, h), dtype=np.float64)
    for j in range(k):
        use = idx[:, j] >= 0
        y[use] += w[use, j, None] * per_pair[use, j]
    return y
