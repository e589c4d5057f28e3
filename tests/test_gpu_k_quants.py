"""GPU parity of the GGUF k-quant linears (q4_k_linear, q5_k_linear, q6_k_linear and their fused
gate_up + SiLU forms) against the CPU oracle: small shapes element by element (several
tiles, ragged tiles, row counts that are not a launch size), the hand-derived
super-blocks, exact-arithmetic inputs bit for bit, a Qwen3-8B FFN in the Q4_K_M mix
(gate_up Q4_K, down Q6_K) and its gate_up in Q5_K at their real sizes with every output
checked, long rows, and
batch invariance (rows of calls with two or more activation rows are bit-identical; one
row runs the one-row kernel where it applies and agrees to float32 reassociation)."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import assert_close, fused_ref_full, linear_ref_full, say, to_dev, torch_dev

pytestmark = pytest.mark.gpu

# bytes per 32 weights (the chunked oracle helpers slice rows with it)
PER32 = {"q4_k": 144 / 8, "q5_k": 176 / 8, "q6_k": 210 / 8}
SB = {"q4_k": 144, "q5_k": 176, "q6_k": 210}
FORMATS = ["q4_k", "q5_k", "q6_k"]


@pytest.fixture(scope="module")
def q8():
    torch, dev = torch_dev()
    import block_quantized_weight_linear_amd as q8mod
    return q8mod, torch, dev


def weight(fmt, seed, n, k, exact=False):
    gen = {"q4_k": wl.q4_k_weight, "q5_k": wl.q5_k_weight, "q6_k": wl.q6_k_weight}[fmt]
    return gen(seed, n, k, exact=exact)[0]


def fns(lib, fmt):
    return getattr(lib, f"{fmt}_linear"), getattr(lib, f"{fmt}_linear_fused_gate_up_silu")


def refs(fmt):
    return getattr(oracle, f"{fmt}_linear_ref"), getattr(oracle, f"fused_gate_up_silu_{fmt}_ref")


SMALL = [(1, 256), (3, 256), (37, 512), (257, 768), (1000, 1024), (513, 3072), (129, 3840), (77, 12288), (64, 2048)]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("n,k", SMALL)
@pytest.mark.parametrize("m", [1, 2, 3, 8, 9, 13, 16, 17])
def test_k_quant_linear_small_vs_oracle(q8, fmt, n, k, m):
    lib, torch, dev = q8
    lin, _ = fns(lib, fmt)
    ref, _ = refs(fmt)
    wb = weight(fmt, 3100 + n + k, n, k)
    x = wl.activations(3200 + m + k, m, k)
    say(f"{fmt}_linear n={n} k={k} m={m}")
    y = lin(to_dev(wb, dev), n, k, to_dev(x, dev)).cpu().numpy()
    assert_close(y, ref(wb, n, k, x), f"{fmt} n={n} k={k} m={m}")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("f,k", [(1, 256), (5, 512), (300, 1024), (129, 3840), (64, 768)])
@pytest.mark.parametrize("m", [1, 4, 8, 11])
def test_k_quant_fused_small_vs_oracle(q8, fmt, f, k, m):
    lib, torch, dev = q8
    _, fused = fns(lib, fmt)
    _, fref = refs(fmt)
    wb = weight(fmt, 3300 + f + k, 2 * f, k)
    x = wl.activations(3400 + m, m, k)
    say(f"{fmt} fused f={f} k={k} m={m}")
    h = fused(to_dev(wb, dev), f, k, to_dev(x, dev)).cpu().numpy()
    assert_close(h, fref(wb, f, k, x), f"{fmt} fused f={f} k={k} m={m}")


def test_k_quant_hand_super_blocks(q8):
    """The hand-derived super-blocks (one K = 256 row each) against activations that pick
    out single weights and weighted sums, every product exact."""
    from golden_io import load_k_quant_cases
    lib, torch, dev = q8
    cases = load_k_quant_cases()
    for fmt in FORMATS:
        mine = [c for c in cases if c["format"] == fmt]
        assert mine
        raw = np.frombuffer(b"".join(c["bytes"] for c in mine), dtype=np.uint8)
        x = np.zeros((3, 256), np.float32)
        x[0] = 1.0
        x[1] = np.arange(256) % 5 - 2
        x[2, 17] = 1.0
        lin, _ = fns(lib, fmt)
        y = lin(to_dev(raw, dev), len(mine), 256, to_dev(x, dev)).cpu().numpy()
        wh = np.array([c["w"] for c in mine], dtype=np.float64)
        assert np.array_equal(y.astype(np.float64), x.astype(np.float64) @ wh.T), fmt


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("n,k,m", [(4096, 1024, 1), (6144, 3840, 8), (999, 256, 33), (2048, 4096, 3),
                                   (16384, 1024, 1)])
def test_k_quant_exact_arithmetic_bit_identical(q8, fmt, n, k, m):
    """d, dmin in {2^-7, 2^-8}, small scales, activations in {-2..2}: every weight and
    every float32 partial sum is a multiple of 2^-8 well inside 2^24 of them, so the
    result is exact in any summation order and must equal the oracle bit for bit."""
    lib, torch, dev = q8
    lin, fused = fns(lib, fmt)
    ref, fref = refs(fmt)
    wb = weight(fmt, 3500 + n, n, k, exact=True)
    x = wl.activations_exact(3600 + m, m, k)
    say(f"{fmt} exact n={n} k={k} m={m}")
    y = lin(to_dev(wb, dev), n, k, to_dev(x, dev)).cpu().numpy()
    assert np.array_equal(y.astype(np.float64), ref(wb, n, k, x))


@pytest.mark.parametrize("fmt", FORMATS)
def test_k_quant_fused_exact_gate_up(q8, fmt):
    """Exact inputs through the fused form: the gate and up sums are exact, so the output
    is SiLU(g) * u of exact g, u, within the float32 epilogue's rounding."""
    lib, torch, dev = q8
    _, fused = fns(lib, fmt)
    _, fref = refs(fmt)
    f, k, m = 1500, 2048, 5
    wb = weight(fmt, 3700, 2 * f, k, exact=True)
    x = wl.activations_exact(3701, m, k)
    h = fused(to_dev(wb, dev), f, k, to_dev(x, dev)).cpu().numpy()
    assert_close(h, fref(wb, f, k, x), f"{fmt} fused exact")


def test_k_quant_qwen3_8b_ffn_full(q8):
    """Qwen3-8B FFN (hidden 4096, intermediate 12288) in the Q4_K_M mix: fused gate_up
    24576 x 4096 in Q4_K, down 4096 x 12288 in Q6_K (and in Q4_K), at m = 1 and 8, every
    output against the oracle."""
    lib, torch, dev = q8
    hid, ff = 4096, 12288
    wg = weight("q4_k", 3800, 2 * ff, hid)
    wgd = to_dev(wg, dev)
    downs = {fmt: weight(fmt, 3801, hid, ff) for fmt in ("q6_k", "q4_k")}
    wg5 = weight("q5_k", 3806, 2 * ff, hid)
    wg5d = to_dev(wg5, dev)
    for m in (1, 8):
        x = wl.activations(3802 + m, m, hid)
        say(f"qwen3-8b q4_k gate_up m={m}")
        h = lib.q4_k_linear_fused_gate_up_silu(wgd, ff, hid, to_dev(x, dev)).cpu().numpy()
        ref = fused_ref_full(wg, ff, hid, x, ref=oracle.fused_gate_up_silu_q4_k_ref, block_bytes=PER32["q4_k"])
        assert_close(h, ref, f"gate_up m={m}")
        say(f"qwen3-8b q5_k gate_up m={m}")
        h5 = lib.q5_k_linear_fused_gate_up_silu(wg5d, ff, hid, to_dev(x, dev)).cpu().numpy()
        ref = fused_ref_full(wg5, ff, hid, x, ref=oracle.fused_gate_up_silu_q5_k_ref, block_bytes=PER32["q5_k"])
        assert_close(h5, ref, f"q5_k gate_up m={m}")
        xh = wl.activations(3804 + m, m, ff)
        for fmt, wd in downs.items():
            say(f"qwen3-8b {fmt} down m={m}")
            lin, _ = fns(lib, fmt)
            ref_fn, _ = refs(fmt)
            y = lin(to_dev(wd, dev), hid, ff, to_dev(xh, dev)).cpu().numpy()
            ref = linear_ref_full(wd, hid, ff, xh, ref=ref_fn, block_bytes=PER32[fmt])
            assert_close(y, ref, f"{fmt} down m={m}")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("n,k", [(4096, 1024), (777, 3840), (12288, 4096), (4096, 12288)])
def test_k_quant_batch_invariance(q8, fmt, n, k):
    """Run to run identical, and every row of a call with two or more activation rows
    bit-identical to the same row of any other such call (the rows kernel's per-output
    order depends only on K).  A one-row call runs the one-row kernel (per-sub-block chains,
    the min / offset terms carried by the activation sums) where it applies, so there rows
    agree to float32 reassociation; fused: the same."""
    lib, torch, dev = q8
    lin, fused = fns(lib, fmt)
    ref_fn, fref = refs(fmt)
    wb = weight(fmt, 3900, n, k)
    wd = to_dev(wb, dev)
    x = wl.activations(3901, 20, k)
    xd = to_dev(x, dev)
    y20 = lin(wd, n, k, xd).cpu().numpy()
    assert np.array_equal(y20, lin(wd, n, k, xd).cpu().numpy())
    for r0, r1 in ((3, 5), (0, 5), (7, 19), (18, 20)):
        assert np.array_equal(lin(wd, n, k, xd[r0:r1].contiguous()).cpu().numpy(), y20[r0:r1]), (r0, r1)
    ref = ref_fn(wb, n, k, x[:3])
    for r in (0, 1, 2):
        y1 = lin(wd, n, k, xd[r:r + 1].contiguous()).cpu().numpy()
        assert np.array_equal(y1, lin(wd, n, k, xd[r:r + 1].contiguous()).cpu().numpy())
        drift = np.max(np.abs(y1[0] - y20[r])) / np.max(np.abs(ref[r]))
        assert drift <= 1e-5, drift
    f = n // 2
    h20 = fused(wd, f, k, xd).cpu().numpy()
    for r0, r1 in ((0, 4), (9, 17)):
        assert np.array_equal(fused(wd, f, k, xd[r0:r1].contiguous()).cpu().numpy(), h20[r0:r1]), (r0, r1)
    h1 = fused(wd, f, k, xd[5:6].contiguous()).cpu().numpy()
    href = fref(wb[:2 * f * (k // 256) * SB[fmt]], f, k, x[5:6])  # the 2f rows the fused call reads
    assert np.max(np.abs(h1[0] - h20[5])) / np.max(np.abs(href)) <= 1e-5


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("n,k,m", [(64, 32768, 1), (70, 65536, 3)])
def test_k_quant_long_rows(q8, fmt, n, k, m):
    lib, torch, dev = q8
    lin, _ = fns(lib, fmt)
    ref, _ = refs(fmt)
    wb = weight(fmt, 4000 + k, n, k)
    x = wl.activations(4001 + m, m, k)
    say(f"{fmt} long rows n={n} k={k} m={m}")
    y = lin(to_dev(wb, dev), n, k, to_dev(x, dev)).cpu().numpy()
    assert_close(y, ref(wb, n, k, x), f"{fmt} long rows k={k} m={m}")


@pytest.mark.parametrize("fmt", FORMATS)
def test_k_quant_binding_rejects_short_weight(q8, fmt):
    lib, torch, dev = q8
    lin, _ = fns(lib, fmt)
    n, k = 8, 512
    wb = weight(fmt, 4100, n, k)
    x = to_dev(wl.activations(4101, 2, k), dev)
    with pytest.raises(ValueError):
        lin(to_dev(wb[:-1], dev), n, k, x)
    assert wb.size == n * (k // 256) * SB[fmt]
