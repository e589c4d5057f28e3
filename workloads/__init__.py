"""Seeded synthetic inputs shared by the tests, the bench and the oracle runs.

This module only draws random numbers and lays them out as bytes; it holds none
of the method's arithmetic (no dequantization, no products, no routing).  Both the
CPU oracle and the HIP library consume what it produces; neither is imported here.

Recipe (the shapes follow the Qwen3 0.6B / 8B / 30B-A3B layers whose linears the
pages describe; the value distributions are fixed here):

* Q8_0 quants ``q``: integers uniform in [-127, 127]; scales ``d``: uniform in
  [1e-3, 2e-2], rounded to binary16 (round to nearest even).
* Activations ``x``: float32 standard normal.
* Router weights: float32 normal with standard deviation 0.02.
* Per-tensor streams come from ``SeedSequence(seed).spawn`` in a fixed order.

A Q8_0 row of length K is K/32 blocks of 34 bytes: a little-endian binary16 scale
followed by 32 int8 quants; rows are contiguous.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

QK = 32
BLOCK_BYTES = 34


# ----------------------------------------------------------------- byte layout


def pack_blocks(q: np.ndarray, d_f16: np.ndarray) -> np.ndarray:
    """Lay int8 quants [N][K] and binary16 scales [N][K/32] out as Q8_0 bytes.

    Returns a flat uint8 array of N*(K/32)*34 bytes.
    """
    q = np.ascontiguousarray(q, dtype=np.int8)
    d_f16 = np.ascontiguousarray(d_f16, dtype=np.float16)
    n, k = q.shape
    nb = k // QK
    if k % QK or d_f16.shape != (n, nb):
        raise ValueError(f"bad shapes q {q.shape} d {d_f16.shape}")
    out = np.empty((n, nb, BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = d_f16.astype("<f2").view(np.uint8).reshape(n, nb, 2)
    out[:, :, 2:] = q.view(np.uint8).reshape(n, nb, QK)
    return out.reshape(-1)


def row_bytes(k: int) -> int:
    return (k // QK) * BLOCK_BYTES


Q4_BLOCK_BYTES = 18


def pack_q4_0(q: np.ndarray, d_f16: np.ndarray) -> np.ndarray:
    """Lay unsigned 4-bit quants [N][K] (values 0..15) and binary16 scales [N][K/32] out as
    GGUF Q4_0 bytes: per block the scale, then byte j = q[j] | q[j + 16] << 4.

    Returns a flat uint8 array of N*(K/32)*18 bytes.
    """
    q = np.ascontiguousarray(q, dtype=np.uint8)
    d_f16 = np.ascontiguousarray(d_f16, dtype=np.float16)
    n, k = q.shape
    nb = k // QK
    if k % QK or d_f16.shape != (n, nb) or q.max(initial=0) > 15:
        raise ValueError(f"bad shapes or values q {q.shape} d {d_f16.shape}")
    qb = q.reshape(n, nb, QK)
    out = np.empty((n, nb, Q4_BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = d_f16.astype("<f2").view(np.uint8).reshape(n, nb, 2)
    out[:, :, 2:] = qb[:, :, :16] | (qb[:, :, 16:] << 4)
    return out.reshape(-1)


Q4_K_BLOCK_BYTES = 144
Q5_K_BLOCK_BYTES = 176
Q6_K_BLOCK_BYTES = 210
QK_K = 256


def pack_q4_k(q, sc, m, d_f16, dmin_f16) -> np.ndarray:
    """Lay GGUF Q4_K super-blocks out as bytes: nibbles q [N][K] (0..15), 6-bit sub-block
    scales sc and mins m [N][K/256][8] (0..63), binary16 d and dmin [N][K/256].

    Per 144-byte super-block: d, dmin, then 12 bytes -- bytes 0..3 hold sc[0..3] in bits
    0-5 and the top two bits of sc[4..7] in bits 6-7, bytes 4..7 the same for m, bytes
    8..11 the low four bits of sc[4..7] (low nibble) and m[4..7] (high nibble) -- then 128
    bytes: byte 32c + i = q[64c + i] | q[64c + 32 + i] << 4.
    """
    q = np.ascontiguousarray(q, dtype=np.uint8)
    n, k = q.shape
    nb = k // QK_K
    sc = np.asarray(sc, dtype=np.uint8).reshape(n, nb, 8)
    m = np.asarray(m, dtype=np.uint8).reshape(n, nb, 8)
    if k % QK_K or q.max(initial=0) > 15 or sc.max(initial=0) > 63 or m.max(initial=0) > 63:
        raise ValueError("bad Q4_K fields")
    out = np.zeros((n, nb, Q4_K_BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = np.asarray(d_f16, dtype="<f2").reshape(n, nb).view(np.uint8).reshape(n, nb, 2)
    out[:, :, 2:4] = np.asarray(dmin_f16, dtype="<f2").reshape(n, nb).view(np.uint8).reshape(n, nb, 2)
    for j in range(4):
        out[:, :, 4 + j] = (sc[:, :, j] & 63) | ((sc[:, :, j + 4] >> 4) << 6)
        out[:, :, 8 + j] = (m[:, :, j] & 63) | ((m[:, :, j + 4] >> 4) << 6)
        out[:, :, 12 + j] = (sc[:, :, j + 4] & 15) | ((m[:, :, j + 4] & 15) << 4)
    qb = q.reshape(n, nb, 4, 2, 32)
    out[:, :, 16:] = (qb[:, :, :, 0, :] | (qb[:, :, :, 1, :] << 4)).reshape(n, nb, 128)
    return out.reshape(-1)


def pack_q5_k(q, sc, m, d_f16, dmin_f16) -> np.ndarray:
    """Lay GGUF Q5_K super-blocks out as bytes: 5-bit quants q [N][K] (0..31), sub-block
    scales and mins as for Q4_K, binary16 d and dmin [N][K/256].

    Per 176-byte super-block: d, dmin, the 12 scale bytes of Q4_K, 32 bytes qh (bit 2c + s
    of byte l is the top bit of quant 64c + 32s + l), then 128 bytes with the low four bits
    as in Q4_K (byte 32c + l = low(q[64c + l]) | low(q[64c + 32 + l]) << 4).
    """
    q = np.ascontiguousarray(q, dtype=np.uint8)
    n, k = q.shape
    nb = k // QK_K
    if k % QK_K or q.max(initial=0) > 31:
        raise ValueError("bad Q5_K fields")
    q4 = pack_q4_k(q & 15, sc, m, d_f16, dmin_f16).reshape(n, nb, Q4_K_BLOCK_BYTES)
    top = (q >> 4).reshape(n, nb, 4, 2, 32).astype(np.uint16)
    qh = np.zeros((n, nb, 32), dtype=np.uint16)
    for c in range(4):
        for half in range(2):
            qh |= top[:, :, c, half, :] << (2 * c + half)
    out = np.zeros((n, nb, Q5_K_BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:16] = q4[:, :, 0:16]
    out[:, :, 16:48] = qh.astype(np.uint8)
    out[:, :, 48:] = q4[:, :, 16:]
    return out.reshape(-1)


def pack_q6_k(q, scales, d_f16) -> np.ndarray:
    """Lay GGUF Q6_K super-blocks out as bytes: 6-bit quants q [N][K] (0..63), int8 scales
    [N][K/256][16], binary16 d [N][K/256].

    Per 210-byte super-block: 128 bytes ql, 64 bytes qh, 16 scales, d.  Weight
    128t + 32k + l (t < 2, k < 4, l < 32) keeps its low four bits in the low (k < 2) or
    high (k >= 2) nibble of ql[64t + l + 32*(k%2)] and its top two bits in bits 2k, 2k+1 of
    qh[32t + l].
    """
    q = np.ascontiguousarray(q, dtype=np.uint8)
    n, k = q.shape
    nb = k // QK_K
    if k % QK_K or q.max(initial=0) > 63:
        raise ValueError("bad Q6_K fields")
    qb = q.reshape(n, nb, 2, 4, 32)                          # t, k, l
    ql = np.zeros((n, nb, 2, 64), dtype=np.uint8)
    qh = np.zeros((n, nb, 2, 32), dtype=np.uint8)
    for kk in range(4):
        low = qb[:, :, :, kk, :] & 15
        seg = slice(32 * (kk % 2), 32 * (kk % 2) + 32)
        ql[..., seg] |= low if kk < 2 else (low << 4)
        qh |= (qb[:, :, :, kk, :] >> 4) << (2 * kk)
    out = np.zeros((n, nb, Q6_K_BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:128] = ql.reshape(n, nb, 128)
    out[:, :, 128:192] = qh.reshape(n, nb, 64)
    out[:, :, 192:208] = np.asarray(scales, dtype=np.int8).reshape(n, nb, 16).view(np.uint8)
    out[:, :, 208:210] = np.asarray(d_f16, dtype="<f2").reshape(n, nb).view(np.uint8).reshape(n, nb, 2)
    return out.reshape(-1)


# ------------------------------------------------------------------ generators


def _rngs(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def q8_weight(seed: int, n: int, k: int, d_lo: float = 1e-3, d_hi: float = 2e-2):
    """Random Q8_0 matrix [n][k]: returns (bytes uint8, q int8 [n][k], d float16 [n][k/32])."""
    rq, rd = _rngs(seed, 2)
    q = rq.integers(-127, 128, size=(n, k), dtype=np.int8)
    d = rd.uniform(d_lo, d_hi, size=(n, k // QK)).astype(np.float16)
    return pack_blocks(q, d), q, d


def q8_weight_exact(seed: int, n: int, k: int):
    """Q8_0 matrix for exact-arithmetic checks: q in [-127, 127], d in {2^-7, 2^-8}.

    With small-integer activations every partial sum is a multiple of 2^-8 far below
    2^24 * 2^-8, so any float32 summation order gives the same, exact result.
    """
    rq, rd = _rngs(seed, 2)
    q = rq.integers(-127, 128, size=(n, k), dtype=np.int8)
    d = np.where(rd.integers(0, 2, size=(n, k // QK)) == 0, 2.0 ** -7, 2.0 ** -8).astype(np.float16)
    return pack_blocks(q, d), q, d


def q4_0_weight(seed: int, n: int, k: int, d_lo: float = 1e-3, d_hi: float = 2e-2):
    """Random Q4_0 matrix [n][k]: returns (bytes uint8, q uint8 [n][k] in 0..15, d float16)."""
    rq, rd = _rngs(seed, 2)
    q = rq.integers(0, 16, size=(n, k), dtype=np.uint8)
    d = rd.uniform(d_lo, d_hi, size=(n, k // QK)).astype(np.float16)
    return pack_q4_0(q, d), q, d


def q4_0_weight_exact(seed: int, n: int, k: int):
    """Q4_0 matrix for exact-arithmetic checks: d in {2^-7, 2^-8} (see q8_weight_exact)."""
    rq, rd = _rngs(seed, 2)
    q = rq.integers(0, 16, size=(n, k), dtype=np.uint8)
    d = np.where(rd.integers(0, 2, size=(n, k // QK)) == 0, 2.0 ** -7, 2.0 ** -8).astype(np.float16)
    return pack_q4_0(q, d), q, d


def q4_k_weight(seed: int, n: int, k: int, exact: bool = False):
    """Random GGUF Q4_K matrix [n][k]: returns (bytes, q, sc, m, d, dmin).  Nibbles
    uniform 0..15, scales and mins uniform 0..63, d and dmin uniform in [2e-5, 2e-4]
    (binary16, some subnormal).  exact: d, dmin in {2^-7, 2^-8} and scales, mins 0..15, so
    with small-integer activations every float32 partial sum is exact."""
    rq, rs, rm, rd, re = _rngs(seed, 5)
    nb = k // QK_K
    q = rq.integers(0, 16, size=(n, k), dtype=np.uint8)
    top = 16 if exact else 64
    sc = rs.integers(0, top, size=(n, nb, 8), dtype=np.uint8)
    mn = rm.integers(0, top, size=(n, nb, 8), dtype=np.uint8)
    if exact:
        d = np.where(rd.integers(0, 2, size=(n, nb)) == 0, 2.0 ** -7, 2.0 ** -8).astype(np.float16)
        dmin = np.where(re.integers(0, 2, size=(n, nb)) == 0, 2.0 ** -7, 2.0 ** -8).astype(np.float16)
    else:
        d = rd.uniform(2e-5, 2e-4, size=(n, nb)).astype(np.float16)
        dmin = re.uniform(2e-5, 2e-4, size=(n, nb)).astype(np.float16)
    return pack_q4_k(q, sc, mn, d, dmin), q, sc, mn, d, dmin


def q5_k_weight(seed: int, n: int, k: int, exact: bool = False):
    """Random GGUF Q5_K matrix [n][k]: returns (bytes, q, sc, m, d, dmin).  Quants uniform
    0..31, scales and mins uniform 0..63, d and dmin uniform in [2e-5, 2e-4] (binary16).
    exact: d, dmin in {2^-7, 2^-8} and scales, mins 0..15."""
    rq, rs, rm, rd, re = _rngs(seed, 5)
    nb = k // QK_K
    q = rq.integers(0, 32, size=(n, k), dtype=np.uint8)
    top = 16 if exact else 64
    sc = rs.integers(0, top, size=(n, nb, 8), dtype=np.uint8)
    mn = rm.integers(0, top, size=(n, nb, 8), dtype=np.uint8)
    if exact:
        d = np.where(rd.integers(0, 2, size=(n, nb)) == 0, 2.0 ** -7, 2.0 ** -8).astype(np.float16)
        dmin = np.where(re.integers(0, 2, size=(n, nb)) == 0, 2.0 ** -7, 2.0 ** -8).astype(np.float16)
    else:
        d = rd.uniform(2e-5, 2e-4, size=(n, nb)).astype(np.float16)
        dmin = re.uniform(2e-5, 2e-4, size=(n, nb)).astype(np.float16)
    return pack_q5_k(q, sc, mn, d, dmin), q, sc, mn, d, dmin


def q6_k_weight(seed: int, n: int, k: int, exact: bool = False):
    """Random GGUF Q6_K matrix [n][k]: returns (bytes, q, scales, d).  Quants uniform
    0..63, scales uniform in [-128, 127], d uniform in [2e-5, 2e-4] (binary16).  exact: d
    in {2^-7, 2^-8}, scales in [-15, 15]."""
    rq, rs, rd = _rngs(seed, 3)
    nb = k // QK_K
    q = rq.integers(0, 64, size=(n, k), dtype=np.uint8)
    if exact:
        scales = rs.integers(-15, 16, size=(n, nb, 16)).astype(np.int8)
        d = np.where(rd.integers(0, 2, size=(n, nb)) == 0, 2.0 ** -7, 2.0 ** -8).astype(np.float16)
    else:
        scales = rs.integers(-128, 128, size=(n, nb, 16)).astype(np.int8)
        d = rd.uniform(2e-5, 2e-4, size=(n, nb)).astype(np.float16)
    return pack_q6_k(q, scales, d), q, scales, d


def activations(seed: int, m: int, k: int) -> np.ndarray:
    """float32 standard-normal activation rows [m][k]."""
    (r,) = _rngs(seed, 1)
    return r.standard_normal((m, k), dtype=np.float32)


def activations_exact(seed: int, m: int, k: int) -> np.ndarray:
    """float32 activation rows with integer values in {-2, ..., 2}."""
    (r,) = _rngs(seed, 1)
    return r.integers(-2, 3, size=(m, k)).astype(np.float32)


def router_weight(seed: int, n_exp: int, h: int, std: float = 0.02) -> np.ndarray:
    """float32 router matrix [n_exp][h] ~ N(0, std^2)."""
    (r,) = _rngs(seed, 1)
    return (r.standard_normal((n_exp, h)) * std).astype(np.float32)


def random_routing(seed: int, m: int, n_exp: int, k: int):
    """Distinct expert ids per token and positive slot weights (not normalized).

    For checking the expert mixture independently of the router.
    """
    r1, r2 = _rngs(seed, 2)
    idx = np.stack([r1.permutation(n_exp)[:k] for _ in range(m)]).astype(np.int32)
    w = r2.uniform(0.05, 1.0, size=(m, k)).astype(np.float32)
    return idx, w


# ------------------------------------------------------------------- workloads


@dataclass(frozen=True)
class Linear:
    name: str
    n: int          # output rows (for gate_up: 2F)
    k: int          # input length
    fused_silu: bool = False

    @property
    def weight_bytes(self) -> int:
        return self.n * row_bytes(self.k)


@dataclass(frozen=True)
class BlockWorkload:
    """The block linears of one decoder layer: QKV, fused gate_up (+SiLU*up), down."""
    name: str
    hidden: int
    qkv_out: int
    ffn: int
    layers: int
    rows: tuple = (1,)
    seed: int = 0
    linears: tuple = field(init=False)

    def __post_init__(self):
        object.__setattr__(self, "linears", (
            Linear("qkv", self.qkv_out, self.hidden),
            Linear("gate_up", 2 * self.ffn, self.hidden, fused_silu=True),
            Linear("down", self.hidden, self.ffn),
        ))

    @property
    def layer_weight_bytes(self) -> int:
        return sum(l.weight_bytes for l in self.linears)


@dataclass(frozen=True)
class MoeWorkload:
    name: str
    hidden: int
    ffn: int
    n_exp: int
    k: int
    tokens: int
    router_std: float = 0.02
    seed: int = 0


# Single linear at the Qwen3-0.6B fused-QKV shape (4096 out, 1024 in), one row.
QWEN3_06B_QKV = Linear("qwen3-0.6b-qkv", 4096, 1024)
# Qwen3-0.6B block linears at M=1; 28 layers (the 0.6B reference config has 28).
QWEN3_06B_BLOCK = BlockWorkload("qwen3-0.6b-block-linears", hidden=1024, qkv_out=4096,
                                ffn=3072, layers=28, rows=(1,), seed=1)
# Qwen3-8B block linears (hidden 4096, 32 q heads + 8 kv heads of 128 -> QKV 6144, FFN 12288).
QWEN3_8B_BLOCK = BlockWorkload("qwen3-8b-block-linears", hidden=4096, qkv_out=6144,
                               ffn=12288, layers=36, rows=(1, 8), seed=2)
# Qwen3-8B gate_up at M=16 (speculative-verify batch) and M=512 (prefill).
QWEN3_8B_GATE_UP = Linear("qwen3-8b-gate-up", 24576, 4096)
GATE_UP_ROWS = (16, 512)
# Qwen3-30B-A3B MoE layer, 16 tokens.
QWEN3_30B_A3B_MOE = MoeWorkload("qwen3-30b-a3b-moe-layer", hidden=2048, ffn=768, n_exp=128,
                                k=8, tokens=16, seed=4)
