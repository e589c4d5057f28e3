"""GPU parity of the integer q8 x q8 path (q8_quantize_act, q8_linear_q8act,
q8_linear_fused_gate_up_silu_q8act) against the CPU oracle.

Codes and scales are integers decided in float32 on both sides: bit-exact.  The
linears are compared element by element on small shapes (many tiles, ragged tails,
row counts that are not a launch size) and on every output of the Qwen3 layer shapes;
inputs whose partial sums are all exact in float32 must match bit for bit.
Invariants: batch invariance and run-to-run determinism.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import assert_close, codes_ref, fused_ref_full, linear_ref_full, say, to_dev, torch_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q8():
    torch, dev = torch_dev()
    import block_quantized_weight_linear_amd as q8mod
    return q8mod, torch, dev


def _special_activations(seed, m, k):
    """Normal rows with planted blocks: all zero, tiny (around the 2^-120 threshold,
    subnormal scales), huge, exact ties of the rounding rule, one-sided signs."""
    x = wl.activations(seed, m, k)
    nb = k // 32
    rng = np.random.default_rng(seed)
    for r in range(m):
        b = rng.permutation(nb)
        x[r, 32 * b[0]:32 * b[0] + 32] = 0.0
        if nb > 1:
            x[r, 32 * b[1]:32 * b[1] + 32] *= np.float32(2.0 ** -121)      # mostly below the threshold
        if nb > 2:
            blk = x[r, 32 * b[2]:32 * b[2] + 32]
            blk *= np.float32(2.0 ** -120) / np.max(np.abs(blk))           # amax exactly 2^-120
        if nb > 3:
            x[r, 32 * b[3]:32 * b[3] + 32] *= np.float32(1e30)
        if nb > 4:  # ties: amax 127 * 2^-4, values (i + 1/2) * 2^-4
            t = (rng.integers(-126, 126, size=32) + 0.5).astype(np.float32)
            t[0] = 127.0
            x[r, 32 * b[4]:32 * b[4] + 32] = t * np.float32(2.0 ** -4)
        if nb > 5:
            x[r, 32 * b[5]:32 * b[5] + 32] = -np.abs(x[r, 32 * b[5]:32 * b[5] + 32])
    return x


@pytest.mark.parametrize("m,k", [(1, 256), (3, 1024), (17, 4096), (5, 12288), (64, 768), (1, 16384)])
def test_quantize_bit_exact(q8, m, k):
    lib, torch, dev = q8
    x = _special_activations(100 + m + k, m, k)
    say(f"quantize m={m} k={k}")
    xq, xd = lib.q8_quantize_act(to_dev(x, dev))
    q_ref, d_ref = oracle.quantize_act_q8_ref(x)
    assert np.array_equal(xq.cpu().numpy(), q_ref)
    assert np.array_equal(xd.cpu().numpy().view(np.uint32), d_ref.view(np.uint32))


def test_quantize_strided_rows_and_hand_cases(q8):
    lib, torch, dev = q8
    from golden_io import load_act_quant_cases
    cases = load_act_quant_cases()
    k = 256
    x = np.zeros((len(cases), k + 64), np.float32)  # rows at a stride of k + 64
    for i, c in enumerate(cases):
        x[i, 96:128] = c["x"]                        # block 3 of the row
    say("quantize hand cases")
    xq, xd = lib.q8_quantize_act(to_dev(x, dev)[:, :k])
    xq, xd = xq.cpu().numpy(), xd.cpu().numpy()
    for i, c in enumerate(cases):
        assert xq[i, 96:128].tolist() == c["q"], c["name"]
        assert float(xd[i, 3]) == c["dx"], c["name"]
        assert np.all(xq[i, :96] == 0) and np.all(xd[i, :3] == 0)


SMALL = [(1, 256), (3, 256), (37, 512), (257, 768), (1000, 1024), (4099, 1024), (513, 3072), (129, 4096),
         (77, 12288), (300, 6144)]


@pytest.mark.parametrize("n,k", SMALL)
@pytest.mark.parametrize("m", [1, 2, 3, 5, 8, 9, 16, 17, 33])
def test_linear_q8act_small_vs_oracle(q8, n, k, m):
    lib, torch, dev = q8
    wb, _, _ = wl.q8_weight(5000 + n + k, n, k)
    qx, dx = oracle.quantize_act_q8_ref(wl.activations(6000 + m + k, m, k))
    say(f"q8_linear_q8act n={n} k={k} m={m}")
    y = lib.q8_linear_q8act(to_dev(wb, dev), n, k, to_dev(qx, dev), to_dev(dx, dev)).cpu().numpy()
    assert_close(y, oracle.q8_linear_codes_ref(wb, n, k, qx, dx), f"q8act n={n} k={k} m={m}")


@pytest.mark.parametrize("f,k", [(1, 256), (5, 512), (300, 1024), (1536, 1024), (129, 4096), (64, 768)])
@pytest.mark.parametrize("m", [1, 4, 8, 13, 16, 19])
def test_fused_q8act_small_vs_oracle(q8, f, k, m):
    lib, torch, dev = q8
    wb, _, _ = wl.q8_weight(7000 + f + k, 2 * f, k)
    qx, dx = oracle.quantize_act_q8_ref(wl.activations(8000 + m, m, k))
    say(f"fused q8act f={f} k={k} m={m}")
    h = lib.q8_linear_fused_gate_up_silu_q8act(to_dev(wb, dev), f, k, to_dev(qx, dev), to_dev(dx, dev))
    assert_close(h.cpu().numpy(), oracle.fused_gate_up_silu_codes_ref(wb, f, k, qx, dx), f"fused q8act f={f} m={m}")


def test_full_int8_range_codes(q8):
    """Codes the quantizer never makes (-128) and arbitrary scales are multiplied exactly."""
    lib, torch, dev = q8
    n, k, m = 513, 1024, 6
    wb, _, _ = wl.q8_weight(9001, n, k)
    rng = np.random.default_rng(9002)
    qx = rng.integers(-128, 128, size=(m, k)).astype(np.int8)
    qx[:, ::7] = -128
    dx = rng.uniform(1e-4, 1e-1, size=(m, k // 32)).astype(np.float32)
    say("q8act full int8 range")
    y = lib.q8_linear_q8act(to_dev(wb, dev), n, k, to_dev(qx, dev), to_dev(dx, dev)).cpu().numpy()
    assert_close(y, oracle.q8_linear_codes_ref(wb, n, k, qx, dx), "full int8 range")


@pytest.mark.parametrize("n,k,m", [(4096, 1024, 1), (6144, 4096, 8), (4096, 12288, 3), (24576, 4096, 16),
                                   (999, 256, 33), (24576, 4096, 1), (24576, 4096, 8), (4096, 12288, 16)])
def test_exact_arithmetic_bit_identical(q8, n, k, m):
    """Codes in [-2, 2], scales 2^-3, weight scales 2^-7 / 2^-8: every float32 partial sum
    is a multiple of 2^-11 below 2^13, so exact in any order."""
    lib, torch, dev = q8
    wb, _, _ = wl.q8_weight_exact(31 + n, n, k)
    qx = wl.activations_exact(32 + m, m, k).astype(np.int8)
    dx = np.full((m, k // 32), 2.0 ** -3, np.float32)
    say(f"q8act exact n={n} k={k} m={m}")
    y = lib.q8_linear_q8act(to_dev(wb, dev), n, k, to_dev(qx, dev), to_dev(dx, dev)).cpu().numpy()
    ref = linear_ref_full(wb, n, k, (qx, dx), ref=codes_ref(oracle.q8_linear_codes_ref))
    assert np.array_equal(y.astype(np.float64), ref), np.max(np.abs(y - ref))


LAYER_LINEARS = [
    ("0.6b qkv", 4096, 1024, False, (1,)),
    ("8b qkv", 6144, 4096, False, (1, 8, 16)),
    ("8b gate_up", 12288, 4096, True, (1, 8, 16)),
    ("8b down", 4096, 12288, False, (1, 8, 16)),
]


@pytest.mark.parametrize("name,n,k,fused,rows", LAYER_LINEARS, ids=[c[0] for c in LAYER_LINEARS])
def test_layer_shapes_full_end_to_end(q8, name, n, k, fused, rows):
    """Quantize on the device (codes bit-exact), then the linear: every output against the
    oracle from the float32 inputs."""
    lib, torch, dev = q8
    wb, _, _ = wl.q8_weight(41, 2 * n if fused else n, k)
    wd = to_dev(wb, dev)
    for m in rows:
        x = wl.activations(42 + m, m, k)
        say(f"{name} q8act m={m}")
        xq, xd = lib.q8_quantize_act(to_dev(x, dev))
        qx, dx = oracle.quantize_act_q8_ref(x)
        assert np.array_equal(xq.cpu().numpy(), qx) and np.array_equal(xd.cpu().numpy(), dx)
        if fused:
            y = lib.q8_linear_fused_gate_up_silu_q8act(wd, n, k, xq, xd).cpu().numpy()
            ref = fused_ref_full(wb, n, k, (qx, dx), ref=codes_ref(oracle.fused_gate_up_silu_codes_ref))
        else:
            y = lib.q8_linear_q8act(wd, n, k, xq, xd).cpu().numpy()
            ref = linear_ref_full(wb, n, k, (qx, dx), ref=codes_ref(oracle.q8_linear_codes_ref))
        assert_close(y, ref, f"{name} q8act m={m} (all {y.size} outputs)")


@pytest.mark.parametrize("n,k", [(4096, 1024), (1024, 3072), (6144, 4096), (777, 12288)])
def test_batch_invariance_and_determinism(q8, n, k):
    """The per-output order depends only on K: any row of any call (1 to 40 rows, in
    16-row launches) is bit-identical to the same row of any other call."""
    lib, torch, dev = q8
    wb, _, _ = wl.q8_weight(51, n, k)
    wd = to_dev(wb, dev)
    qx, dx = oracle.quantize_act_q8_ref(wl.activations(52, 40, k))
    qd, dd = to_dev(qx, dev), to_dev(dx, dev)
    say(f"q8act batch invariance n={n} k={k}")
    y40 = lib.q8_linear_q8act(wd, n, k, qd, dd).cpu().numpy()
    assert np.array_equal(y40, lib.q8_linear_q8act(wd, n, k, qd, dd).cpu().numpy())
    for r0, r1 in ((0, 1), (0, 2), (3, 7), (5, 13), (0, 16), (20, 37), (39, 40)):
        ym = lib.q8_linear_q8act(wd, n, k, qd[r0:r1].contiguous(), dd[r0:r1].contiguous()).cpu().numpy()
        assert np.array_equal(ym, y40[r0:r1]), (r0, r1)
    f = n // 2
    h40 = lib.q8_linear_fused_gate_up_silu_q8act(wd, f, k, qd, dd).cpu().numpy()
    for r0, r1 in ((0, 1), (2, 11), (30, 40)):
        hm = lib.q8_linear_fused_gate_up_silu_q8act(wd, f, k, qd[r0:r1].contiguous(), dd[r0:r1].contiguous())
        assert np.array_equal(hm.cpu().numpy(), h40[r0:r1]), (r0, r1)


def test_zero_rows_and_outputs(q8):
    lib, torch, dev = q8
    k = 512
    wb, _, _ = wl.q8_weight(61, 8, k)
    qx = torch.empty((0, k), dtype=torch.int8, device=dev)
    dx = torch.empty((0, k // 32), dtype=torch.float32, device=dev)
    assert lib.q8_linear_q8act(to_dev(wb, dev), 8, k, qx, dx).shape == (0, 8)
    xq, xd = lib.q8_quantize_act(torch.empty((0, k), dtype=torch.float32, device=dev))
    assert xq.shape == (0, k) and xd.shape == (0, k // 32)


def test_q8act_graph_replay_matches_eager(q8):
    """Quantize + the int8-dot linears captured in one HIP graph: every replay, with eager
    work in between, gives the eager result bit for bit."""
    lib, torch, dev = q8
    k, n, f = 1024, 4096, 1536
    wq = to_dev(wl.q8_weight(91, n, k)[0], dev)
    wg = to_dev(wl.q8_weight(92, 2 * f, k)[0], dev)
    for m in (1, 9):
        x = to_dev(wl.activations(93 + m, m, k), dev)
        xq = torch.empty((m, k), dtype=torch.int8, device=dev)
        xd = torch.empty((m, k // 32), device=dev)
        y = torch.empty((m, n), device=dev)
        h = torch.empty((m, f), device=dev)

        def step():
            lib.q8_quantize_act(x, xq, xd)
            lib.q8_linear_q8act(wq, n, k, xq, xd, out=y)
            lib.q8_linear_fused_gate_up_silu_q8act(wg, f, k, xq, xd, out=h)

        step()
        torch.cuda.synchronize()
        ref = [t.clone() for t in (xq, xd, y, h)]
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                step()
        for rep in range(4):
            for t in (xd, y, h):
                t.fill_(float("nan"))
            xq.fill_(0)
            g.replay()
            torch.cuda.synchronize()
            for got, want in zip((xq, xd, y, h), ref):
                assert torch.equal(got, want), (m, rep)
            step()
            torch.cuda.synchronize()


@pytest.mark.parametrize("n,k,m", [(64, 32768, 1), (100, 65536, 5)])
def test_q8act_long_rows(q8, n, k, m):
    lib, torch, dev = q8
    wb, _, _ = wl.q8_weight(2100 + k, n, k)
    x = wl.activations(2101 + m, m, k)
    xq, xd = lib.q8_quantize_act(to_dev(x, dev))
    qx, dx = oracle.quantize_act_q8_ref(x)
    assert np.array_equal(xq.cpu().numpy(), qx)
    y = lib.q8_linear_q8act(to_dev(wb, dev), n, k, xq, xd).cpu().numpy()
    assert_close(y, oracle.q8_linear_codes_ref(wb, n, k, qx, dx), f"q8act long rows k={k} m={m}")
