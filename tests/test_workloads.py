"""The seeded input generators: determinism, ranges and byte layout (CPU only)."""

import struct

import numpy as np

import workloads as wl
from golden_io import half_bits_to_fraction


def test_deterministic():
    a = wl.q8_weight(5, 8, 256)
    b = wl.q8_weight(5, 8, 256)
    assert all(np.array_equal(u, v) for u, v in zip(a, b))
    assert not np.array_equal(wl.q8_weight(6, 8, 256)[0], a[0])
    assert np.array_equal(wl.activations(1, 2, 64), wl.activations(1, 2, 64))


def test_ranges():
    _, q, d = wl.q8_weight(9, 64, 1024)
    assert q.min() >= -127 and q.max() <= 127
    df = d.astype(np.float64)
    assert df.min() >= 1e-3 * (1 - 2 ** -11) and df.max() <= 2e-2 * (1 + 2 ** -11)
    _, qe, de = wl.q8_weight_exact(9, 16, 256)
    assert set(np.unique(de.astype(np.float64))) <= {2.0 ** -7, 2.0 ** -8}
    xe = wl.activations_exact(3, 4, 256)
    assert set(np.unique(xe)) <= {-2.0, -1.0, 0.0, 1.0, 2.0}
    wr = wl.router_weight(4, 128, 2048)
    assert wr.dtype == np.float32 and abs(float(wr.std()) - 0.02) < 5e-4


def test_layout_matches_struct_reading():
    """Each 34-byte block is <binary16 d><32 x int8 q>, blocks along K, rows contiguous."""
    n, k = 3, 96
    buf, q, d = wl.q8_weight(11, n, k)
    assert buf.dtype == np.uint8 and buf.size == n * (k // 32) * 34
    raw = buf.tobytes()
    for r in range(n):
        for b in range(k // 32):
            off = (r * (k // 32) + b) * 34
            (bits,) = struct.unpack_from("<H", raw, off)
            qs = struct.unpack_from("<32b", raw, off + 2)
            assert half_bits_to_fraction(bits) == half_bits_to_fraction(int(d.view(np.uint16)[r, b]))
            assert list(qs) == q[r, 32 * b:32 * b + 32].tolist()


def test_routing_generator():
    idx, w = wl.random_routing(2, 16, 128, 8)
    assert idx.shape == (16, 8) and w.shape == (16, 8)
    for row in idx:
        assert len(set(row.tolist())) == 8 and row.min() >= 0 and row.max() < 128
    assert w.min() > 0


def test_workload_sizes():
    assert wl.QWEN3_06B_QKV.weight_bytes == 4_456_448
    assert wl.QWEN3_06B_BLOCK.layer_weight_bytes == 14_483_456
    assert wl.QWEN3_06B_BLOCK.layer_weight_bytes * 28 == 405_536_768
    assert wl.QWEN3_8B_BLOCK.layer_weight_bytes == 187_170_816
    assert wl.QWEN3_8B_GATE_UP.weight_bytes == 106_954_752


def test_k_quant_generators_sizes_and_ranges():
    wb, q, sc, mn, d, dmin = wl.q4_k_weight(1, 3, 512)
    assert wb.size == 3 * 2 * 144 and q.max() <= 15 and sc.max() <= 63 and mn.max() <= 63
    wb6, q6, s6, d6 = wl.q6_k_weight(2, 3, 512)
    assert wb6.size == 3 * 2 * 210 and q6.max() <= 63 and s6.dtype == np.int8
    we, _, sce, _, de, dme = wl.q4_k_weight(3, 2, 256, exact=True)
    assert sce.max() <= 15 and set(np.unique(de.astype(np.float64))) <= {2.0 ** -7, 2.0 ** -8}
