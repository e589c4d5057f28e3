"""GPU parity of q4_0_linear and q4_0_linear_fused_gate_up_silu (GGUF Q4_0 weights)
against the CPU oracle: small shapes element by element (tiles, ragged chunks, row
counts that are not a launch size), the Gemma 4 12B FFN shape at its real size (every output), hand
blocks, exact-arithmetic inputs bit for bit, batch invariance (one-row calls are their own
kernel class, as for Q8_0)."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import assert_close, fused_ref_full, linear_ref_full, say, to_dev, torch_dev

pytestmark = pytest.mark.gpu

Q4_BLOCK = 18


@pytest.fixture(scope="module")
def q8():
    torch, dev = torch_dev()
    import block_quantized_weight_linear_amd as q8mod
    return q8mod, torch, dev


def q4_rows(wbytes, k, rows):
    rb = (k // 32) * Q4_BLOCK
    return np.ascontiguousarray(wbytes.reshape(-1, rb)[np.asarray(rows)]).reshape(-1)


SMALL = [(1, 256), (3, 256), (37, 512), (257, 768), (1000, 1024), (513, 3072), (129, 3840), (77, 12288), (64, 2048)]


@pytest.mark.parametrize("n,k", SMALL)
@pytest.mark.parametrize("m", [1, 2, 3, 8, 9, 13, 16, 17])
def test_q4_0_linear_small_vs_oracle(q8, n, k, m):
    lib, torch, dev = q8
    wb, _, _ = wl.q4_0_weight(1100 + n + k, n, k)
    x = wl.activations(1200 + m + k, m, k)
    say(f"q4_0_linear n={n} k={k} m={m}")
    y = lib.q4_0_linear(to_dev(wb, dev), n, k, to_dev(x, dev)).cpu().numpy()
    assert_close(y, oracle.q4_0_linear_ref(wb, n, k, x), f"q4_0 n={n} k={k} m={m}")


@pytest.mark.parametrize("f,k", [(1, 256), (5, 512), (300, 1024), (129, 3840), (64, 768)])
@pytest.mark.parametrize("m", [1, 4, 8, 11])
def test_q4_0_fused_small_vs_oracle(q8, f, k, m):
    lib, torch, dev = q8
    wb, _, _ = wl.q4_0_weight(1300 + f + k, 2 * f, k)
    x = wl.activations(1400 + m, m, k)
    say(f"q4_0 fused f={f} k={k} m={m}")
    h = lib.q4_0_linear_fused_gate_up_silu(to_dev(wb, dev), f, k, to_dev(x, dev)).cpu().numpy()
    assert_close(h, oracle.fused_gate_up_silu_q4_0_ref(wb, f, k, x), f"q4_0 fused f={f} k={k} m={m}")


# One row on matrices with K <= 4096 and at least 16 row groups per CU (256 CUs): the
# one-row kernel with Q4_0 pairs; 1, 2 and 4 rows per wave slot group, ragged row groups.
@pytest.mark.parametrize("n,k,fused", [(4096, 3840, False), (8192, 2048, False), (4100, 4096, False),
                                       (4096, 3840, True), (16400, 768, True)])
def test_q4_0_one_row_large_vs_oracle(q8, n, k, fused):
    lib, torch, dev = q8
    wb, _, _ = wl.q4_0_weight(2300 + n + k, 2 * n if fused else n, k)
    x = wl.activations(2400 + k, 1, k)
    say(f"q4_0 one row n={n} k={k} fused={fused}")
    if fused:
        h = lib.q4_0_linear_fused_gate_up_silu(to_dev(wb, dev), n, k, to_dev(x, dev)).cpu().numpy()
        assert_close(h, oracle.fused_gate_up_silu_q4_0_ref(wb, n, k, x), f"q4_0 one row fused f={n} k={k}")
    else:
        y = lib.q4_0_linear(to_dev(wb, dev), n, k, to_dev(x, dev)).cpu().numpy()
        assert_close(y, oracle.q4_0_linear_ref(wb, n, k, x), f"q4_0 one row n={n} k={k}")


def test_q4_0_hand_blocks(q8):
    """The hand-derived blocks, each the first block of a K = 256 row padded with zero
    blocks (d = 0), against activations chosen so that every product is exact."""
    from golden_io import load_q4_0_cases
    lib, torch, dev = q8
    cases = load_q4_0_cases()
    k = 256
    zero = bytes(Q4_BLOCK)
    raw = np.frombuffer(b"".join(c["bytes"] + zero * 7 for c in cases), dtype=np.uint8)
    x = np.zeros((2, k), np.float32)
    x[0, :32] = 1.0
    x[1, :32] = np.arange(32) % 5 - 2
    y = lib.q4_0_linear(to_dev(raw, dev), len(cases), k, to_dev(x, dev)).cpu().numpy()
    wh = np.array([c["w"] for c in cases])
    assert np.array_equal(y.astype(np.float64), x[:, :32].astype(np.float64) @ wh.T)


@pytest.mark.parametrize("n,k,m", [(4096, 1024, 1), (6144, 3840, 8), (999, 256, 33), (2048, 12288, 3),
                                   (16384, 1024, 1), (4096, 3840, 1)])
def test_q4_0_exact_arithmetic_bit_identical(q8, n, k, m):
    """Scales 2^-7 / 2^-8, activations in {-2..2}: every float32 partial sum is exact."""
    lib, torch, dev = q8
    wb, _, _ = wl.q4_0_weight_exact(1500 + n, n, k)
    x = wl.activations_exact(1600 + m, m, k)
    say(f"q4_0 exact n={n} k={k} m={m}")
    y = lib.q4_0_linear(to_dev(wb, dev), n, k, to_dev(x, dev)).cpu().numpy()
    assert np.array_equal(y.astype(np.float64), oracle.q4_0_linear_ref(wb, n, k, x))


def test_q4_0_gemma4_12b_ffn_full(q8):
    """Gemma 4 12B FFN (hidden 3840, intermediate 15360): fused gate_up 30720 x 3840 and
    down 3840 x 15360 at m = 1 and 8, every output against the oracle."""
    lib, torch, dev = q8
    hid, ff = 3840, 15360
    wg, _, _ = wl.q4_0_weight(1700, 2 * ff, hid)
    wd, _, _ = wl.q4_0_weight(1701, hid, ff)
    wgd, wdd = to_dev(wg, dev), to_dev(wd, dev)
    for m in (1, 8):
        x = wl.activations(1702 + m, m, hid)
        say(f"gemma-4-12b q4_0 gate_up m={m}")
        h = lib.q4_0_linear_fused_gate_up_silu(wgd, ff, hid, to_dev(x, dev)).cpu().numpy()
        ref = fused_ref_full(wg, ff, hid, x, ref=oracle.fused_gate_up_silu_q4_0_ref, block_bytes=Q4_BLOCK)
        assert_close(h, ref, f"gate_up m={m}")
        xh = wl.activations(1704 + m, m, ff)
        y = lib.q4_0_linear(wdd, hid, ff, to_dev(xh, dev)).cpu().numpy()
        ref = linear_ref_full(wd, hid, ff, xh, ref=oracle.q4_0_linear_ref, block_bytes=Q4_BLOCK)
        assert_close(y, ref, f"down m={m}")


@pytest.mark.parametrize("n,k", [(4096, 1024), (777, 3840), (15360, 3840)])
def test_q4_0_batch_invariance(q8, n, k):
    """Run to run identical.  Rows of any call with 2 or more activation rows are
    bit-identical to the same rows of any other such call.  A one-row call on a large
    matrix with K <= 4096 (here 15360 x 3840, and 7680 fused outputs) runs the one-row
    kernel (per-block sums, the -8 offset carried by the block's activation sum), whose
    summation order differs, so there rows agree to float32 reassociation, as for Q8_0; on
    the smaller shapes the one-row call is bit-identical as well."""
    lib, torch, dev = q8
    wb, _, _ = wl.q4_0_weight(1800, n, k)
    wd = to_dev(wb, dev)
    x = wl.activations(1801, 20, k)
    xd = to_dev(x, dev)
    y20 = lib.q4_0_linear(wd, n, k, xd).cpu().numpy()
    assert np.array_equal(y20, lib.q4_0_linear(wd, n, k, xd).cpu().numpy())
    for r0, r1 in ((3, 5), (0, 5), (7, 19)):
        assert np.array_equal(lib.q4_0_linear(wd, n, k, xd[r0:r1].contiguous()).cpu().numpy(), y20[r0:r1]), (r0, r1)
    ref = oracle.q4_0_linear_ref(wb, n, k, x[:3])
    for r in (0, 1, 2):
        y1 = lib.q4_0_linear(wd, n, k, xd[r:r + 1].contiguous()).cpu().numpy()
        assert np.array_equal(y1, lib.q4_0_linear(wd, n, k, xd[r:r + 1].contiguous()).cpu().numpy())
        drift = np.max(np.abs(y1[0] - y20[r])) / np.max(np.abs(ref[r]))
        assert drift <= 1e-5, drift
    # fused: the same properties
    f = n // 2
    h20 = lib.q4_0_linear_fused_gate_up_silu(wd, f, k, xd).cpu().numpy()
    assert np.array_equal(lib.q4_0_linear_fused_gate_up_silu(wd, f, k, xd[:4].contiguous()).cpu().numpy(), h20[:4])
    h1 = lib.q4_0_linear_fused_gate_up_silu(wd, f, k, xd[5:6].contiguous()).cpu().numpy()
    href = oracle.fused_gate_up_silu_q4_0_ref(q4_rows(wb, k, np.arange(2 * f)), f, k, x[5:6])
    assert np.max(np.abs(h1[0] - h20[5])) / np.max(np.abs(href)) <= 1e-5


@pytest.mark.parametrize("n,k,m", [(64, 32768, 1), (70, 65536, 3)])
def test_q4_0_long_rows(q8, n, k, m):
    lib, torch, dev = q8
    wb, _, _ = wl.q4_0_weight(2200 + k, n, k)
    x = wl.activations(2201 + m, m, k)
    y = lib.q4_0_linear(to_dev(wb, dev), n, k, to_dev(x, dev)).cpu().numpy()
    assert_close(y, oracle.q4_0_linear_ref(wb, n, k, x), f"q4_0 long rows k={k} m={m}")
