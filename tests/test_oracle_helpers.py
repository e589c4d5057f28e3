"""The test helpers that run the oracle at full size (row chunks, expert-grouped calls)
give the oracle's own results: checked on the CPU against the unchunked oracle calls."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import codes_ref, fused_ref_full, linear_ref_full, moe_mixture_grouped_ref


@pytest.mark.parametrize("n,k,m,chunk", [(1000, 256, 3, 128), (77, 512, 1, 10), (300, 1024, 5, 300)])
def test_chunked_linear_equals_oracle(n, k, m, chunk):
    wb, _, _ = wl.q8_weight(11 + n, n, k)
    x = wl.activations(12 + m, m, k)
    np.testing.assert_allclose(linear_ref_full(wb, n, k, x, chunk=chunk), oracle.q8_linear_ref(wb, n, k, x),
                               rtol=1e-13, atol=1e-13)
    f = n // 2
    wf = wb[:2 * f * (k // 32) * 34]
    np.testing.assert_allclose(fused_ref_full(wf, f, k, x, chunk=chunk), oracle.fused_gate_up_silu_ref(wf, f, k, x),
                               rtol=1e-13, atol=1e-13)


def test_chunked_codes_and_q4_0_equal_oracle():
    n, k, m = 130, 512, 4
    wb, _, _ = wl.q8_weight(21, n, k)
    qx, dx = oracle.quantize_act_q8_ref(wl.activations(22, m, k))
    np.testing.assert_allclose(linear_ref_full(wb, n, k, (qx, dx), chunk=17, ref=codes_ref(oracle.q8_linear_codes_ref)),
                               oracle.q8_linear_codes_ref(wb, n, k, qx, dx), rtol=1e-13, atol=1e-13)
    w4, _, _ = wl.q4_0_weight(23, 2 * n, k)
    x = wl.activations(24, m, k)
    np.testing.assert_allclose(
        fused_ref_full(w4, n, k, x, chunk=33, ref=oracle.fused_gate_up_silu_q4_0_ref, block_bytes=18),
        oracle.fused_gate_up_silu_q4_0_ref(w4, n, k, x), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("m,e,k,f,h,drop", [(9, 5, 3, 256, 256, False), (20, 4, 2, 256, 512, True)])
def test_grouped_mixture_equals_oracle(m, e, k, f, h, drop):
    gu = np.concatenate([wl.q8_weight(30 + i, 2 * f, h)[0] for i in range(e)])
    dn = np.concatenate([wl.q8_weight(60 + i, h, f)[0] for i in range(e)])
    x = wl.activations(90, m, h)
    idx, w = wl.random_routing(91, m, e, k)
    w = w.astype(np.float64)
    if drop:  # slots dropped by a top-p cut: expert -1, weight 0
        idx[::3, k - 1] = -1
        w[::3, k - 1] = 0.0
    got = moe_mixture_grouped_ref(gu, dn, e, f, h, x, idx, w)
    want = oracle.moe_mixture_ref(gu, dn, e, f, h, x, idx, w)
    # batched and one-row float64 products may round differently in the last bits
    assert oracle.rel_err_row_max(got, want) <= 1e-13
