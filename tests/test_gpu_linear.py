"""GPU parity of q8_linear and q8_linear_fused_gate_up_silu against the CPU oracle.

Small shapes (many tiles and ragged tails) and the Qwen3 layer shapes at their real
sizes (the oracle run in row chunks) are compared element by element with the full
oracle; only the matrices too tall for the streaming form are compared on sampled
output rows.  Exact-arithmetic inputs (every partial
sum representable in float32) must match bit for bit.  Invariants: batch invariance,
run-to-run determinism, scale doubling, sign symmetry, zero blocks, one-hot gathers.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import TOL, assert_close, fused_ref_full, linear_ref_full, row_slice, sample_rows, say, to_dev, torch_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q8():
    torch, dev = torch_dev()
    import block_quantized_weight_linear_amd as q8mod
    return q8mod, torch, dev


SMALL = [(1, 256), (3, 256), (37, 512), (257, 768), (1000, 1024), (4099, 1024), (513, 3072), (129, 4096),
         (77, 12288), (64, 2048), (300, 6144)]


@pytest.mark.parametrize("n,k", SMALL)
@pytest.mark.parametrize("m", [1, 2, 3, 5, 8, 9, 12, 13, 16, 17, 33])
def test_linear_small_vs_oracle(q8, n, k, m):
    lib, torch, dev = q8
    wb, _, _ = wl.q8_weight(1000 + n + k, n, k)
    x = wl.activations(2000 + m + k, m, k)
    say(f"q8_linear n={n} k={k} m={m}")
    y = lib.q8_linear(to_dev(wb, dev), n, k, to_dev(x, dev)).cpu().numpy()
    assert_close(y, oracle.q8_linear_ref(wb, n, k, x), f"linear n={n} k={k} m={m}")


@pytest.mark.parametrize("f,k", [(1, 256), (5, 512), (300, 1024), (1536, 1024), (129, 4096), (64, 768)])
@pytest.mark.parametrize("m", [1, 4, 8, 11, 16, 19])
def test_fused_small_vs_oracle(q8, f, k, m):
    lib, torch, dev = q8
    wb, _, _ = wl.q8_weight(3000 + f + k, 2 * f, k)
    x = wl.activations(4000 + m, m, k)
    say(f"fused f={f} k={k} m={m}")
    h = lib.q8_linear_fused_gate_up_silu(to_dev(wb, dev), f, k, to_dev(x, dev)).cpu().numpy()
    assert_close(h, oracle.fused_gate_up_silu_ref(wb, f, k, x), f"fused f={f} k={k} m={m}")


# One activation row on matrices with at least 16 row groups per CU: the one-row kernel's
# 8-wave configuration (non-temporal weight copies), 1, 2 and 3 rounds of 64 pairs, ragged
# pair counts (K = 4352: 68 pairs; K = 6144: 96), plain and fused; full oracle.
@pytest.mark.parametrize("n,k,fused", [(6144, 4096, False), (4096, 12288, False), (2048, 8192, False),
                                       (5000, 6144, False), (4096, 4096, True), (2048, 8192, True),
                                       (2100, 4352, True),
                                       # four rounds (12288 < K <= 16384), small and large matrices,
                                       # plain and fused, K = 12544 leaves a ragged last round
                                       (4096, 16384, False), (100, 16384, False), (4100, 12544, False),
                                       (77, 12544, False), (4096, 16384, True), (96, 16384, True),
                                       (4099, 12544, True), (33, 12544, True)])
def test_one_row_large_vs_oracle(q8, n, k, fused):
    lib, torch, dev = q8
    wb, _, _ = wl.q8_weight(5000 + n + k, 2 * n if fused else n, k)
    x = wl.activations(6000 + k, 1, k)
    say(f"one row n={n} k={k} fused={fused}")
    if fused:
        h = lib.q8_linear_fused_gate_up_silu(to_dev(wb, dev), n, k, to_dev(x, dev)).cpu().numpy()
        assert_close(h, oracle.fused_gate_up_silu_ref(wb, n, k, x), f"one row fused f={n} k={k}")
    else:
        y = lib.q8_linear(to_dev(wb, dev), n, k, to_dev(x, dev)).cpu().numpy()
        assert_close(y, oracle.q8_linear_ref(wb, n, k, x), f"one row n={n} k={k}")


# ------------------------------------------------------------ real layer shapes

LAYER_LINEARS = [
    # (name, n, k, fused, rows)   n = outputs (F for fused)
    ("0.6b qkv", 4096, 1024, False, (1,)),
    ("0.6b gate_up", 3072, 1024, True, (1,)),
    ("0.6b down", 1024, 3072, False, (1,)),
    ("8b qkv", 6144, 4096, False, (1, 8)),
    ("8b gate_up", 12288, 4096, True, (1, 8)),
    ("8b down", 4096, 12288, False, (1, 8)),
    ("8b gate_up plain", 24576, 4096, False, (16,)),
]


@pytest.mark.parametrize("name,n,k,fused,rows", LAYER_LINEARS, ids=[c[0] for c in LAYER_LINEARS])
def test_layer_shapes_full(q8, name, n, k, fused, rows):
    """Every output of the Qwen3 layer linears at their real sizes against the oracle."""
    lib, torch, dev = q8
    w_rows = 2 * n if fused else n
    wb, _, _ = wl.q8_weight(11, w_rows, k)
    wd = to_dev(wb, dev)
    for m in rows:
        x = wl.activations(12 + m, m, k)
        say(f"{name} m={m}")
        fn = lib.q8_linear_fused_gate_up_silu if fused else lib.q8_linear
        y = fn(wd, n, k, to_dev(x, dev)).cpu().numpy()
        ref = fused_ref_full(wb, n, k, x) if fused else linear_ref_full(wb, n, k, x)
        assert_close(y, ref, f"{name} m={m} (all {y.size} outputs)")


# Exact-arithmetic inputs at the layer shapes (every output, bit for bit), on both one-row
# configurations, the rows kernel at 2..16 rows and its persistent walk over many tiles.
@pytest.mark.parametrize("n,k,m,fused", [(4096, 1024, 1, False), (6144, 4096, 8, False), (4096, 12288, 3, False),
                                         (24576, 4096, 16, False), (1024, 3072, 1, False), (999, 256, 33, False),
                                         (6144, 4096, 1, False), (4096, 12288, 1, False), (4096, 12288, 8, False),
                                         (6144, 4096, 16, False), (24576, 4096, 1, False), (12288, 4096, 1, True),
                                         (12288, 4096, 8, True), (12288, 4096, 16, True), (4096, 16384, 1, False)])
def test_exact_arithmetic_bit_identical(q8, n, k, m, fused):
    """Integer activations in [-2, 2], scales 2^-7 / 2^-8: every float32 partial sum is exact,
    so every linear output equals the oracle bit for bit.  The fused form's SiLU makes its
    outputs inexact; there the gate and up sums are checked exactly through the plain call
    on the same matrix, and the fused outputs to the float32 tolerance."""
    lib, torch, dev = q8
    w_rows = 2 * n if fused else n
    wb, _, _ = wl.q8_weight_exact(21 + n, w_rows, k)
    x = wl.activations_exact(22 + m, m, k)
    say(f"exact n={n} k={k} m={m} fused={fused}")
    wd, xd = to_dev(wb, dev), to_dev(x, dev)
    y = lib.q8_linear(wd, w_rows, k, xd).cpu().numpy()
    ref = linear_ref_full(wb, w_rows, k, x)
    assert np.array_equal(y.astype(np.float64), ref), np.max(np.abs(y - ref))
    if fused:
        h = lib.q8_linear_fused_gate_up_silu(wd, n, k, xd).cpu().numpy()
        assert_close(h, oracle.silu_ref(ref[:, :n]) * ref[:, n:], f"exact fused f={n} m={m}")


# Many more row tiles than resident blocks with a short K: the persistent walk over many
# tiles per block of the rows kernel and of its matrix-core form (9..16 rows), every output
# against the oracle.
@pytest.mark.parametrize("n,k,m,fused", [(40000, 256, 8, False), (40000, 256, 16, False), (20000, 512, 8, True),
                                         (20000, 512, 3, True), (40000, 256, 1, False), (20000, 512, 1, True),
                                         (20000, 512, 13, True), (30000, 1024, 10, False)])
def test_many_tiles_vs_oracle(q8, n, k, m, fused):
    lib, torch, dev = q8
    w_rows = 2 * n if fused else n
    wb, _, _ = wl.q8_weight(1200 + n + m, w_rows, k)
    x = wl.activations(1201 + m, m, k)
    say(f"many tiles n={n} k={k} m={m} fused={fused}")
    fn = lib.q8_linear_fused_gate_up_silu if fused else lib.q8_linear
    y = fn(to_dev(wb, dev), n, k, to_dev(x, dev)).cpu().numpy()
    ref = fused_ref_full(wb, n, k, x) if fused else linear_ref_full(wb, n, k, x)
    assert_close(y, ref, f"many tiles n={n} k={k} m={m} fused={fused}")


# ------------------------------------------------------------------- invariants


@pytest.mark.parametrize("n,k", [(4096, 1024), (1024, 3072), (6144, 4096), (777, 12288)])
def test_batch_invariance_and_determinism(q8, n, k):
    """Run-to-run bit-identical.  Rows of any call with 2..16 activation rows (and the
    16-row chunks of larger calls) are bit-identical to the same rows of any other such
    call; a one-row call uses the single-row kernel, whose summation order differs, so
    there rows agree to float32 reassociation (the batch-kernel threshold behaviour of
    "14. Model families and example applications", section 14.2)."""
    lib, torch, dev = q8
    wb, _, _ = wl.q8_weight(31, n, k)
    wd = to_dev(wb, dev)
    x = wl.activations(32, 40, k)
    xd = to_dev(x, dev)
    say(f"batch invariance n={n} k={k}")
    y40 = lib.q8_linear(wd, n, k, xd).cpu().numpy()
    y40b = lib.q8_linear(wd, n, k, xd).cpu().numpy()
    assert np.array_equal(y40, y40b)  # run to run
    for m in (2, 5, 8, 10, 13, 16):
        ym = lib.q8_linear(wd, n, k, xd[:m].contiguous()).cpu().numpy()
        assert np.array_equal(ym, y40[:m]), m
    for r in (3, 17, 38):
        y2 = lib.q8_linear(wd, n, k, xd[r:r + 2].contiguous()).cpu().numpy()
        assert np.array_equal(y2, y40[r:r + 2]), r
    ref = oracle.q8_linear_ref(wb, n, k, x[:4])
    for r in (0, 1, 2, 3):
        y1 = lib.q8_linear(wd, n, k, xd[r:r + 1].contiguous()).cpu().numpy()
        y1b = lib.q8_linear(wd, n, k, xd[r:r + 1].contiguous()).cpu().numpy()
        assert np.array_equal(y1, y1b)
        drift = np.max(np.abs(y1[0] - y40[r])) / np.max(np.abs(ref[r]))
        assert drift <= 1e-5, drift
    # fused: same properties
    f = n // 2
    h40 = lib.q8_linear_fused_gate_up_silu(wd, f, k, xd).cpu().numpy()
    for m in (2, 9, 12, 15):
        hm = lib.q8_linear_fused_gate_up_silu(wd, f, k, xd[:m].contiguous()).cpu().numpy()
        assert np.array_equal(hm, h40[:m]), m
    h1 = lib.q8_linear_fused_gate_up_silu(wd, f, k, xd[5:6].contiguous()).cpu().numpy()
    href = oracle.fused_gate_up_silu_ref(row_slice(wb, k, np.arange(2 * f)), f, k, x[5:6])
    assert np.max(np.abs(h1[0] - h40[5])) / np.max(np.abs(href)) <= 1e-5


@pytest.mark.parametrize("n,k", [(300, 20480), (64, 4096), (1000, 16640), (6144, 4096)])
def test_rows_kernels_agree_bit_for_bit(q8, n, k):
    """2..16 activation rows agree bit for bit whatever the call's row count, plain and
    fused: at K = 4096 on the streaming form (activation rows padded to 4, 8, 12 or 16), at
    larger K on the float32 rows kernel (up to 8 rows) and its matrix-core form (9..16 rows,
    padded to 12 or 16), which give the same bits.  One row with K past the one-row kernel
    also runs the float32 rows kernel; it is checked to float32 reassociation only, the
    class the interface promises for one row."""
    lib, torch, dev = q8
    wb, _, _ = wl.q8_weight(2300 + n, n, k)
    x = wl.activations(2301, 16, k)
    wd, xd = to_dev(wb, dev), to_dev(x, dev)
    say(f"rows kernels agree n={n} k={k}")
    y16 = lib.q8_linear(wd, n, k, xd).cpu().numpy()
    for m in (13, 10, 5):
        ym = lib.q8_linear(wd, n, k, xd[:m].contiguous()).cpu().numpy()
        assert np.array_equal(ym, y16[:m]), m
    f = n // 2
    h16 = lib.q8_linear_fused_gate_up_silu(wd, f, k, xd).cpu().numpy()
    for m in (11, 7):
        hm = lib.q8_linear_fused_gate_up_silu(wd, f, k, xd[:m].contiguous()).cpu().numpy()
        assert np.array_equal(hm, h16[:m]), m
    if k > 16384:  # one row past the one-row kernel: the float32 rows kernel
        for r in (0, 9, 15):
            y1 = lib.q8_linear(wd, n, k, xd[r:r + 1].contiguous()).cpu().numpy()
            assert np.max(np.abs(y1[0] - y16[r])) <= 1e-5 * np.max(np.abs(y16[r])), r
            h1 = lib.q8_linear_fused_gate_up_silu(wd, f, k, xd[r:r + 1].contiguous()).cpu().numpy()
            assert np.max(np.abs(h1[0] - h16[r])) <= 1e-5 * np.max(np.abs(h16[r])), r


def stream_form_applies(n_out, k, silu, cu_count=256):
    """Whether a call takes the streaming rows form: K <= 4096 and its LDS (two ring slots
    of 4352 bytes per wave and row group, plus the chunk sums of every item of a block at
    16 rows and one block per CU) fits in 160 KB; the host-side rule, restated."""
    p = k // 64
    nc = (p + 15) // 16
    if nc > 4:
        return False
    rg = 2 if silu else 1
    items = -(-((n_out + 3) // 4) // cu_count)
    return nc * 2 * rg * 4352 + items * nc * rg * 4 * 16 * 4 <= 160 * 1024


def test_rows_kernels_on_matrices_too_tall_for_the_streaming_form(q8):
    """640,000 output rows at K = 256 (174 MB of Q8_0): the streaming form's LDS does not
    fit, so up to 8 rows run the float32 rows kernel and 9..16 its matrix-core form; the
    two give the same bits (one fma per weight and row in the same order), checked against
    each other and against the oracle on sampled outputs."""
    lib, torch, dev = q8
    n, k = 640_000, 256
    assert not stream_form_applies(n, k, False)
    wb, _, _ = wl.q8_weight(2400, n, k)
    x = wl.activations(2401, 16, k)
    wd, xd = to_dev(wb, dev), to_dev(x, dev)
    say(f"too tall for the streaming form n={n} k={k}")
    y16 = lib.q8_linear(wd, n, k, xd).cpu().numpy()
    for m in (13, 8, 5, 2):
        ym = lib.q8_linear(wd, n, k, xd[:m].contiguous()).cpu().numpy()
        assert np.array_equal(ym, y16[:m]), m
    rows = sample_rows(n, 256, seed=7)
    ref = oracle.q8_linear_ref(row_slice(wb, k, rows), len(rows), k, x)
    assert_close(y16[:, rows], ref, f"too tall n={n} k={k} sampled outputs")


def test_scale_doubling_sign_and_zero_blocks(q8):
    lib, torch, dev = q8
    n, k, m = 2048, 2048, 4
    _, q, d = wl.q8_weight(41, n, k)
    x = wl.activations(42, m, k)
    xd = to_dev(x, dev)
    y = lib.q8_linear(to_dev(wl.pack_blocks(q, d), dev), n, k, xd).cpu().numpy()
    d2 = (d.astype(np.float32) * 2).astype(np.float16)
    y2 = lib.q8_linear(to_dev(wl.pack_blocks(q, d2), dev), n, k, xd).cpu().numpy()
    assert np.array_equal(y2, 2 * y)
    yx = lib.q8_linear(to_dev(wl.pack_blocks(q, d), dev), n, k, to_dev(2 * x, dev)).cpu().numpy()
    assert np.array_equal(yx, 2 * y)
    yn = lib.q8_linear(to_dev(wl.pack_blocks(-q, d), dev), n, k, xd).cpu().numpy()
    assert np.array_equal(yn, -y)
    mask = np.random.default_rng(1).random(d.shape) < 0.3
    d0 = d.copy()
    d0[mask] = 0
    q0 = q.copy().reshape(n, k // 32, 32)
    q0[mask] = 0
    ya = lib.q8_linear(to_dev(wl.pack_blocks(q, d0), dev), n, k, xd).cpu().numpy()
    yb = lib.q8_linear(to_dev(wl.pack_blocks(q0.reshape(n, k), d), dev), n, k, xd).cpu().numpy()
    assert np.array_equal(ya, yb)
    assert_close(ya, oracle.q8_linear_ref(wl.pack_blocks(q, d0), n, k, x), "zero blocks")
    yz = lib.q8_linear(to_dev(wl.pack_blocks(q, np.zeros_like(d)), dev), n, k, xd).cpu().numpy()
    assert np.all(yz == 0)


def test_one_hot_gather(q8):
    lib, torch, dev = q8
    n, k, m = 1000, 4096, 3
    perm = np.random.default_rng(5).permutation(k)[:n]
    q = np.zeros((n, k), np.int8)
    q[np.arange(n), perm] = 1
    d = np.ones((n, k // 32), np.float16)
    x = wl.activations(51, m, k)
    y = lib.q8_linear(to_dev(wl.pack_blocks(q, d), dev), n, k, to_dev(x, dev)).cpu().numpy()
    assert np.array_equal(y, x[:, perm])


def test_hand_blocks_on_gpu(q8):
    """The hand-derived cases, padded to K = 256 with zero blocks and zero activations."""
    from golden_io import load_linear_cases
    lib, torch, dev = q8
    for c in load_linear_cases():
        k0, n = c["k"], c["n"]
        k = 256
        rb0 = (k0 // 32) * 34
        rows = np.frombuffer(c["w"], np.uint8).reshape(n, rb0)
        pad = np.zeros((n, (k - k0) // 32 * 34), np.uint8)
        wb = np.concatenate([rows, pad], axis=1).reshape(-1)
        x = np.zeros((len(c["x"]), k), np.float32)
        x[:, :k0] = np.array(c["x"], np.float32)
        y = lib.q8_linear(to_dev(wb, dev), n, k, to_dev(x, dev)).cpu().numpy()
        want = np.array([[float(v) for v in r] for r in c["y"]])
        np.testing.assert_allclose(y, want, rtol=2e-7, atol=0, err_msg=c["name"])


# ------------------------------------------------------------------- edge cases


def test_edge_sizes_and_strides(q8):
    lib, torch, dev = q8
    k = 512
    wb, _, _ = wl.q8_weight(61, 10, k)
    wd = to_dev(wb, dev)
    # no rows
    y = lib.q8_linear(wd, 10, k, torch.empty((0, k), dtype=torch.float32, device=dev))
    assert tuple(y.shape) == (0, 10)
    # no outputs
    y = lib.q8_linear(wd, 0, k, to_dev(wl.activations(1, 2, k), dev))
    assert tuple(y.shape) == (2, 0)
    # strided x and y: x rows inside a wider buffer, y written into a wider buffer
    xb = to_dev(wl.activations(62, 5, k + 64), dev)
    xs = xb[:, :k]
    out = torch.full((5, 32), 7.0, dtype=torch.float32, device=dev)
    lib.q8_linear(wd, 10, k, xs, out=out[:, :10])
    o = out.cpu().numpy()
    assert np.all(o[:, 10:] == 7.0)
    assert_close(o[:, :10], oracle.q8_linear_ref(wb, 10, k, xs.cpu().numpy()), "strided")


def test_binding_rejects_bad_arguments(q8):
    """The binding refuses, before any launch, tensors the kernels would read or write
    past: a short weight, an output with too few rows or columns, a transposed output,
    overlapping rows; the C ABI refuses what it can see (K not a multiple of 256)."""
    lib, torch, dev = q8
    wb, _, _ = wl.q8_weight(71, 8, 256)
    wd = to_dev(wb, dev)
    x2 = torch.zeros((2, 256), dtype=torch.float32, device=dev)
    with pytest.raises(ValueError):
        lib.q8_linear(wd, 8, 256, torch.zeros((1, 128), dtype=torch.float32, device=dev))
    with pytest.raises(lib.Q8Error):
        lib.q8_linear(wd[:0], 8, 96, torch.zeros((1, 96), dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):  # one output row for two activation rows
        lib.q8_linear(wd, 8, 256, x2, out=torch.empty((1, 8), device=dev))
    with pytest.raises(ValueError):  # transposed output (column stride 2)
        lib.q8_linear(wd, 8, 256, x2, out=torch.empty((8, 2), device=dev).t())
    with pytest.raises(ValueError):  # too few columns
        lib.q8_linear(wd, 8, 256, x2, out=torch.empty((2, 7), device=dev))
    with pytest.raises(ValueError):  # weight holds 7 rows, the call names 8
        lib.q8_linear(wd[:7 * 8 * 34], 8, 256, x2)
    with pytest.raises(ValueError):  # fused: 2f rows needed
        lib.q8_linear_fused_gate_up_silu(wd, 8, 256, x2)
    with pytest.raises(ValueError):  # overlapping activation rows
        lib.q8_linear(wd, 8, 256, torch.zeros(512, device=dev).as_strided((2, 256), (128, 1)))
    with pytest.raises(ValueError):
        lib.q4_0_linear(wd[:8 * 8 * 18 - 1], 8, 256, x2)
    with pytest.raises(ValueError):
        lib.q8_quantize_act(x2, xq=torch.empty((1, 256), dtype=torch.int8, device=dev))
    xq, xdd = lib.q8_quantize_act(x2)
    with pytest.raises(ValueError):
        lib.q8_linear_q8act(wd, 8, 256, xq, xdd, out=torch.empty((1, 8), device=dev))
    xr = torch.zeros((3, 256), dtype=torch.float32, device=dev)
    wr = torch.zeros((8, 256), dtype=torch.float32, device=dev)
    with pytest.raises(ValueError):  # idx_out with fewer than k columns
        lib.moe_route_topk(xr, wr, 4, idx_out=torch.empty((3, 3), dtype=torch.int32, device=dev))
    with pytest.raises(ValueError):  # w_out with fewer rows
        lib.moe_route_topk(xr, wr, 4, w_out=torch.empty((2, 4), device=dev))
    gu = torch.zeros(4 * 2 * 256 * 8 * 34, dtype=torch.uint8, device=dev)
    dn = torch.zeros(4 * 256 * 8 * 34, dtype=torch.uint8, device=dev)
    idx = torch.zeros((3, 2), dtype=torch.int32, device=dev)
    wts = torch.zeros((3, 2), device=dev)
    with pytest.raises(ValueError):  # expert stack shorter than n_exp experts
        lib.q8_moe_grouped_linear(gu[:-1], dn, 4, 256, 256, xr, idx, wts)
    with pytest.raises(ValueError):
        lib.q8_moe_grouped_linear(gu, dn, 4, 256, 256, xr, idx, wts, out=torch.empty((3, 255), device=dev))
    with pytest.raises(ValueError):
        lib.q8_moe_grouped_linear(gu, dn, 4, 256, 256, xr, idx, wts[:2])
    y = lib.q8_moe_grouped_linear(gu, dn, 4, 256, 256, xr, idx, wts)  # well-formed: runs
    assert tuple(y.shape) == (3, 256)


def test_graph_replay_matches_eager(q8):
    """The three block linears captured in one HIP graph: every replay, with eager work
    and synchronizations in between, gives the eager result bit for bit."""
    lib, torch, dev = q8
    k, nq, f = 1024, 4096, 3072
    wq, _, _ = wl.q8_weight(81, nq, k)
    wg, _, _ = wl.q8_weight(82, 2 * f, k)
    wdn, _, _ = wl.q8_weight(83, k, f)
    wq, wg, wdn = to_dev(wq, dev), to_dev(wg, dev), to_dev(wdn, dev)
    for m in (1, 3):
        x = to_dev(wl.activations(84 + m, m, k), dev)
        yq = torch.empty((m, nq), device=dev)
        h = torch.empty((m, f), device=dev)
        yd = torch.empty((m, k), device=dev)

        def step():
            lib.q8_linear(wq, nq, k, x, out=yq)
            lib.q8_linear_fused_gate_up_silu(wg, f, k, x, out=h)
            lib.q8_linear(wdn, k, f, h, out=yd)

        step()
        torch.cuda.synchronize()
        ref = [t.clone() for t in (yq, h, yd)]
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                step()
        for rep in range(4):
            for t in (yq, h, yd):
                t.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            for got, want in zip((yq, h, yd), ref):
                assert torch.equal(got, want), (m, rep)
            step()  # eager work between replays
            torch.cuda.synchronize()


# ------------------------------------------------------- prefill (bf16 matrix cores)

PREFILL_TOL = 2e-2   # bf16 operands, float32 accumulation


# With at least as many 128 x 256 tiles as CUs (256 on the MI355X) the prefill runs 8-wave
# 128 x 256 tiles: (32768, 256, 256) and the ragged (33000, 256, 300) take that path there;
# the smaller shapes take the 4-wave 128 x 128 / 128 x 64 tiles.
@pytest.mark.parametrize("n,k,m", [(300, 1024, 256), (129, 512, 300), (1024, 4096, 512), (77, 3072, 257),
                                   (520, 256, 1000), (32768, 256, 256), (33000, 256, 300),
                                   (1024, 12288, 256)])  # the 8B down's K, 32-column waves
def test_prefill_vs_oracle(q8, n, k, m):
    lib, torch, dev = q8
    wb, _, _ = wl.q8_weight(91 + n, n, k)
    x = wl.activations(92 + m, m, k)
    say(f"prefill n={n} k={k} m={m}")
    y = lib.q8_linear(to_dev(wb, dev), n, k, to_dev(x, dev)).cpu().numpy()
    assert_close(y, oracle.q8_linear_ref(wb, n, k, x), f"prefill n={n} k={k} m={m}", tol=PREFILL_TOL)
    # with both operands rounded to bf16 first, only float32 accumulation error remains
    diag = oracle.q8_linear_bf16_operands_ref(wb, n, k, x)
    assert_close(y, diag, f"prefill vs bf16-operand oracle n={n} m={m}", tol=1e-4)


@pytest.mark.parametrize("f,k,m", [(64, 1024, 256), (200, 512, 300), (1536, 2048, 512), (16384, 256, 256),
                                   (16500, 256, 260)])
def test_prefill_fused_vs_oracle(q8, f, k, m):
    lib, torch, dev = q8
    wb, _, _ = wl.q8_weight(93 + f, 2 * f, k)
    x = wl.activations(94 + m, m, k)
    say(f"prefill fused f={f} k={k} m={m}")
    h = lib.q8_linear_fused_gate_up_silu(to_dev(wb, dev), f, k, to_dev(x, dev)).cpu().numpy()
    assert_close(h, oracle.fused_gate_up_silu_ref(wb, f, k, x), f"prefill fused f={f} m={m}", tol=PREFILL_TOL)
    gu = oracle.q8_linear_bf16_operands_ref(wb, 2 * f, k, x)
    diag = oracle.silu_ref(gu[:, :f]) * gu[:, f:]
    assert_close(h, diag, f"prefill fused vs bf16-operand oracle f={f}", tol=1e-4)


def test_prefill_qwen3_8b_gate_up_full(q8):
    """Qwen3-8B gate_up 24576x4096 at M=512 (the prefill configuration): every output, plain
    and fused, against the oracle (and against the bf16-operand oracle)."""
    lib, torch, dev = q8
    n, k, m = 24576, 4096, 512
    wb, _, _ = wl.q8_weight(11, n, k)
    x = wl.activations(95, m, k)
    wd, xd = to_dev(wb, dev), to_dev(x, dev)
    say("prefill 8b gate_up m=512")
    y = lib.q8_linear(wd, n, k, xd).cpu().numpy()
    assert_close(y, linear_ref_full(wb, n, k, x, chunk=4096), "8b gate_up m=512", tol=PREFILL_TOL)
    diag = linear_ref_full(wb, n, k, x, chunk=4096, ref=oracle.q8_linear_bf16_operands_ref)
    assert_close(y, diag, "8b gate_up m=512 vs bf16-operand oracle", tol=1e-4)
    h = lib.q8_linear_fused_gate_up_silu(wd, n // 2, k, xd).cpu().numpy()
    assert_close(h, oracle.silu_ref(diag[:, :n // 2]) * diag[:, n // 2:], "8b fused gate_up m=512 vs bf16-operand",
                 tol=1e-4)
    assert_close(h, fused_ref_full(wb, n // 2, k, x, chunk=4096), "8b fused gate_up m=512", tol=PREFILL_TOL)


@pytest.mark.parametrize("n,k,m", [(4096, 1024, 256), (1000, 4096, 512), (32768, 256, 256), (24576, 4096, 512)])
def test_prefill_exact_arithmetic(q8, n, k, m):
    """Integer activations and scales 2^-7 / 2^-8: bf16 holds every operand exactly and every
    float32 partial sum is exact, so the matrix-core result equals the oracle bit for bit."""
    lib, torch, dev = q8
    wb, _, _ = wl.q8_weight_exact(96 + n, n, k)
    x = wl.activations_exact(97 + m, m, k)
    say(f"prefill exact n={n} k={k} m={m}")
    y = lib.q8_linear(to_dev(wb, dev), n, k, to_dev(x, dev)).cpu().numpy()
    assert np.array_equal(y.astype(np.float64), linear_ref_full(wb, n, k, x, chunk=4096))


@pytest.mark.parametrize("n,k,m", [(64, 32768, 1), (33, 20480, 1), (64, 32768, 3), (130, 65536, 2)])
def test_long_rows(q8, n, k, m):
    """K beyond what the one-row kernel keeps in registers (more than 4 pair rounds per
    lane): one row falls back to the rows kernel; long rows also in the fused form."""
    lib, torch, dev = q8
    wb, _, _ = wl.q8_weight(1900 + n + k, n, k)
    x = wl.activations(1901 + m, m, k)
    say(f"long rows n={n} k={k} m={m}")
    y = lib.q8_linear(to_dev(wb, dev), n, k, to_dev(x, dev)).cpu().numpy()
    assert_close(y, oracle.q8_linear_ref(wb, n, k, x), f"long rows n={n} k={k} m={m}")
    f = n // 2
    wf = row_slice(wb, k, np.arange(2 * f))
    h = lib.q8_linear_fused_gate_up_silu(to_dev(wf, dev), f, k, to_dev(x, dev)).cpu().numpy()
    assert_close(h, oracle.fused_gate_up_silu_ref(wf, f, k, x), f"long rows fused f={f} k={k} m={m}")
