"""Helpers shared by the GPU parity tests (device transfers, sampled oracle rows)."""

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
