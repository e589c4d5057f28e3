"""Plain, slow CPU reference (float64) for the Q8_0 block-quantized weight linear.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports this module: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may call it.  It shares no code with the HIP library (no kernels, headers,
helpers, tables or pre/post-processing) and imports nothing from it.

What it follows (sources are the four pages describing the fucina engine):

* "14. Model families and example applications", section 14.1 (Conventions shared
  by every family): LinearWeight keeps the GGUF dtype resident and the quant forms,
  Q8_0 among them, run packed kernels with no global dequantization at load; q/k/v
  are fused into one QKV matrix and gate/up into one gate_up matrix.
* Same page, section 14.2 (Qwen3 - dense and MoE): SwiGLU FFN; the MoE FFN routes
  with a softmax top-k (``routerTopK`` with ``normalize_selected = norm_topk_prob``,
  default true) and runs the router-weighted SwiGLU mixture (``moeSwiGluFfnSeq``).
* Same page, section 14.4 (Gemma 4 - text + MoE, "MoE expert kernels"): the combine
  keeps each token's summation order fixed.

Every step is the plain definition written out in float64: parse the blocks,
dequantize exactly, multiply with a library matmul, apply the elementwise
epilogue.  No blocking, fusion or reordering.

Readings taken where the pages are silent:

* Q8_0 byte layout: the GGUF Q8_0 block -- one little-endian IEEE binary16 scale
  ``d`` followed by 32 signed 8-bit quants ``q``, 34 bytes; blocks run along K and
  rows are contiguous.  The pages name Q8_0 but never spell the layout out.
* Dequantization is ``w = d * q`` (no zero point, no minimum).  It is exact in
  float64: an 11-bit significand times an 8-bit integer.
* Orientation: ``y[m, n] = sum_k x[m, k] * W[n, k]`` (N outputs, K inputs, GGUF rows
  with K innermost).
* gate_up rows are concatenated: gate rows ``[0, F)`` then up rows ``[F, 2F)``.
* SiLU is ``g * sigmoid(g)``.
* Top-k ties go to the lower expert index; the output is ordered by descending
  probability (equivalently, descending logit).
* The MoE hidden activation ``SiLU(gate) * up`` stays un-requantized.

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py`` against
hand-computed block values (``tests/golden/``), exact rational brute force, closed
forms, invariants and library routines.
"""

from __future__ import annotations

import math

import numpy as np

QK8_0 = 32                 # quants per block
Q8_0_BLOCK_BYTES = 34      # 2-byte binary16 scale + 32 int8 quants

# One GGUF Q8_0 block, read as a packed record (no padding: itemsize 34).
_Q8_0_RECORD = np.dtype([("d", "<f2"), ("qs", "i1", (QK8_0,))])
assert _Q8_0_RECORD.itemsize == Q8_0_BLOCK_BYTES


# --------------------------------------------------------------------------- Q8_0


def q8_0_row_bytes(k: int) -> int:
    """Bytes in one Q8_0 row of length k."""
    if k % QK8_0:
        raise ValueError(f"K={k} is not a multiple of {QK8_0}")
    return (k // QK8_0) * Q8_0_BLOCK_BYTES


def parse_q8_0(buf, n_rows: int, k: int):
    """Split a Q8_0 byte stream into its scales and quants, both as float64.

    Returns ``d`` of shape (n_rows, k/32) and ``q`` of shape (n_rows, k/32, 32).
    Both conversions are exact (binary16 -> float64, int8 -> float64).
    """
    raw = np.frombuffer(memoryview(buf).cast("B"), dtype=np.uint8)
    need = n_rows * q8_0_row_bytes(k)
    if raw.size != need:
        raise ValueError(f"Q8_0 buffer has {raw.size} bytes, expected {need}")
    rec = raw.view(_Q8_0_RECORD).reshape(n_rows, k // QK8_0)
    d = rec["d"].astype(np.float64)
    q = rec["qs"].astype(np.float64)
    return d, q


def dequantize_q8_0(buf, n_rows: int, k: int) -> np.ndarray:
    """W[n, 32*b + i] = d[n, b] * q[n, b, i] in float64 (exact)."""
    d, q = parse_q8_0(buf, n_rows, k)
    w = d[:, :, None] * q
    return w.reshape(n_rows, k)


# --------------------------------------------------------------------------- Q4_0
#
# The DGX Spark README (Features; Models) names Q4_0 among the formats read directly by
# the quantized GEMV/GEMM (the Gemma 4 QAT checkpoints), and "14. Model families and
# example applications" section 14.1 says the other ggml quant forms run their own
# packed kernels; neither spells the layout out.  Reading: the GGUF Q4_0 block -- a
# little-endian binary16 scale d, then 16 bytes; weight j (0..15) is the low nibble of
# byte j and weight j + 16 its high nibble, both unsigned 0..15; w = d * (q - 8).  18
# bytes per 32 weights, blocks along K, rows contiguous.

QK4_0 = 32
Q4_0_BLOCK_BYTES = 18
_Q4_0_RECORD = np.dtype([("d", "<f2"), ("qs", "u1", (QK4_0 // 2,))])
assert _Q4_0_RECORD.itemsize == Q4_0_BLOCK_BYTES


def q4_0_row_bytes(k: int) -> int:
    """Bytes in one Q4_0 row of length k."""
    if k % QK4_0:
        raise ValueError(f"K={k} is not a multiple of {QK4_0}")
    return (k // QK4_0) * Q4_0_BLOCK_BYTES


def parse_q4_0(buf, n_rows: int, k: int):
    """Scales d (n_rows, k/32) and unsigned quants q (n_rows, k/32, 32), as float64."""
    raw = np.frombuffer(memoryview(buf).cast("B"), dtype=np.uint8)
    need = n_rows * q4_0_row_bytes(k)
    if raw.size != need:
        raise ValueError(f"Q4_0 buffer has {raw.size} bytes, expected {need}")
    rec = raw.view(_Q4_0_RECORD).reshape(n_rows, k // QK4_0)
    d = rec["d"].astype(np.float64)
    qs = rec["qs"]
    q = np.empty((n_rows, k // QK4_0, QK4_0), dtype=np.float64)
    q[:, :, :16] = qs & 0x0F
    q[:, :, 16:] = qs >> 4
    return d, q


def dequantize_q4_0(buf, n_rows: int, k: int) -> np.ndarray:
    """W[n, 32*b + i] = d[n, b] * (q[n, b, i] - 8) in float64 (exact)."""
    d, q = parse_q4_0(buf, n_rows, k)
    return (d[:, :, None] * (q - 8.0)).reshape(n_rows, k)


def q4_0_linear_ref(w_q4, n: int, k: int, x) -> np.ndarray:
    """y[m, n] = sum_k x[m, k] * W[n, k] with W the dequantized Q4_0 matrix (float64)."""
    return np.asarray(x, dtype=np.float64) @ dequantize_q4_0(w_q4, n, k).T


def fused_gate_up_silu_q4_0_ref(w_gate_up_q4, f: int, k: int, x) -> np.ndarray:
    """SiLU(x . W_gate^T) * (x . W_up^T) from one Q4_0 [2f][k] matrix, gate rows first."""
    y = q4_0_linear_ref(w_gate_up_q4, 2 * f, k, x)
    return silu_ref(y[:, :f]) * y[:, f:]


# ----------------------------------------------------------- Q4_K, Q5_K, Q6_K
#
# "14. Model families and example applications" section 14.1 says the ggml quant forms
# Q4_K, Q5_K and Q6_K run their own packed kernels, and the DGX Spark README (Features)
# lists Q4_K and Q6_K among the formats its GEMV reads directly; neither page spells the
# layouts out.  Reading: the GGUF k-quant super-blocks of 256 weights.
#
# Q4_K, 144 bytes: binary16 d, binary16 dmin, 12 bytes of packed 6-bit sub-block scales
# and mins, 128 bytes of 4-bit quants.  Sub-block j (weights 32j .. 32j+31) has scale
# sc[j] and min m[j]: for j < 4, sc = byte[j] & 63 and m = byte[j+4] & 63; for j >= 4 the
# low four bits come from byte[j+4] (low nibble for sc, high nibble for m) and the top two
# bits from bits 6-7 of byte[j-4] (sc) or byte[j] (m).  Weight 64c + i (i < 32) is the low
# nibble of quant byte 32c + i, weight 64c + 32 + i its high nibble;
# w = d * sc[j] * q - dmin * m[j].
#
# Q5_K, 176 bytes: binary16 d, binary16 dmin, the 12 scale/min bytes of Q4_K (same
# packing), 32 bytes qh, 128 bytes of 4-bit quants.  Weight 64c + 32s + l (c < 4, s < 2,
# l < 32) has the 5-bit quant whose low four bits are nibble s (low for s = 0) of quant
# byte 32c + l and whose top bit is bit 2c + s of qh[l]; it is in sub-block j = 2c + s;
# w = d * sc[j] * q - dmin * m[j].  (Section 14.1 names Q5_K with Q4_K and Q6_K; the same
# reading of the GGUF layout.)
#
# Q6_K, 210 bytes: 128 bytes ql, 64 bytes qh, 16 int8 scales, binary16 d.  Weights run in
# two halves of 128; in half t, weight 128t + 32k + l (k < 4, l < 32) has the 6-bit quant
# whose low four bits are the low (k < 2) or high (k >= 2) nibble of ql[64t + l + 32*(k%2)]
# and whose top two bits are bits 2k, 2k+1 of qh[32t + l]; weight i uses scale i // 16;
# w = d * scale * (q - 32).

QK_K = 256
Q4_K_BLOCK_BYTES = 144
Q5_K_BLOCK_BYTES = 176
Q6_K_BLOCK_BYTES = 210
_Q4_K_RECORD = np.dtype([("d", "<f2"), ("dmin", "<f2"), ("scales", "u1", (12,)), ("qs", "u1", (QK_K // 2,))])
_Q6_K_RECORD = np.dtype([("ql", "u1", (QK_K // 2,)), ("qh", "u1", (QK_K // 4,)), ("scales", "i1", (QK_K // 16,)),
                         ("d", "<f2")])
_Q5_K_RECORD = np.dtype([("d", "<f2"), ("dmin", "<f2"), ("scales", "u1", (12,)), ("qh", "u1", (QK_K // 8,)),
                         ("qs", "u1", (QK_K // 2,))])
assert _Q4_K_RECORD.itemsize == Q4_K_BLOCK_BYTES and _Q6_K_RECORD.itemsize == Q6_K_BLOCK_BYTES
assert _Q5_K_RECORD.itemsize == Q5_K_BLOCK_BYTES


def _k_records(buf, n_rows: int, k: int, record, block_bytes: int):
    if k % QK_K:
        raise ValueError(f"K={k} is not a multiple of {QK_K}")
    raw = np.frombuffer(memoryview(buf).cast("B"), dtype=np.uint8)
    need = n_rows * (k // QK_K) * block_bytes
    if raw.size != need:
        raise ValueError(f"buffer has {raw.size} bytes, expected {need}")
    return raw.view(record).reshape(n_rows, k // QK_K)


def q4_k_scale_min(scales):
    """The eight 6-bit (scale, min) pairs of Q4_K super-blocks: scales [..., 12] bytes ->
    (sc [..., 8], m [..., 8]) as integers 0..63."""
    b = np.asarray(scales, dtype=np.int64)
    sc = np.empty(b.shape[:-1] + (8,), dtype=np.int64)
    m = np.empty_like(sc)
    for j in range(4):
        sc[..., j] = b[..., j] & 63
        m[..., j] = b[..., j + 4] & 63
    for j in range(4, 8):
        sc[..., j] = (b[..., j + 4] & 0x0F) | ((b[..., j - 4] >> 6) << 4)
        m[..., j] = (b[..., j + 4] >> 4) | ((b[..., j] >> 6) << 4)
    return sc, m


def dequantize_q4_k(buf, n_rows: int, k: int) -> np.ndarray:
    """W[n, 256b + i] of a GGUF Q4_K matrix in float64 (exact: each weight is a difference of
    two products of at most 21 significant bits)."""
    rec = _k_records(buf, n_rows, k, _Q4_K_RECORD, Q4_K_BLOCK_BYTES)
    d = rec["d"].astype(np.float64)
    dmin = rec["dmin"].astype(np.float64)
    sc, m = q4_k_scale_min(rec["scales"])                       # [n][nb][8]
    qs = rec["qs"].astype(np.int64).reshape(n_rows, k // QK_K, 4, 32)
    q = np.empty((n_rows, k // QK_K, 4, 2, 32), dtype=np.int64)  # chunk c, sub-block 2c + s
    q[:, :, :, 0, :] = qs & 0x0F
    q[:, :, :, 1, :] = qs >> 4
    q = q.reshape(n_rows, k // QK_K, 8, 32)                    # sub-block j = 2c + s
    w = (d[:, :, None, None] * sc[:, :, :, None]) * q - (dmin[:, :, None, None] * m[:, :, :, None])
    return w.reshape(n_rows, -1)


def dequantize_q5_k(buf, n_rows: int, k: int) -> np.ndarray:
    """W[n, 256b + i] of a GGUF Q5_K matrix in float64 (exact: products of at most 22
    significant bits)."""
    rec = _k_records(buf, n_rows, k, _Q5_K_RECORD, Q5_K_BLOCK_BYTES)
    nb = k // QK_K
    d = rec["d"].astype(np.float64)
    dmin = rec["dmin"].astype(np.float64)
    sc, m = q4_k_scale_min(rec["scales"])                       # [n][nb][8]
    qs = rec["qs"].astype(np.int64).reshape(n_rows, nb, 4, 32)  # chunk c, byte l
    qh = rec["qh"].astype(np.int64)                             # [n][nb][32], byte l
    q5 = np.empty((n_rows, nb, 4, 2, 32), dtype=np.int64)        # chunk c, half s, l
    for c in range(4):
        for half in range(2):
            low4 = (qs[:, :, c, :] >> (4 * half)) & 0x0F
            top = (qh >> (2 * c + half)) & 1
            q5[:, :, c, half, :] = low4 + 16 * top
    q5 = q5.reshape(n_rows, nb, 8, 32)                          # sub-block j = 2c + s
    w = (d[:, :, None, None] * sc[:, :, :, None]) * q5 - (dmin[:, :, None, None] * m[:, :, :, None])
    return w.reshape(n_rows, -1)


def dequantize_q6_k(buf, n_rows: int, k: int) -> np.ndarray:
    """W[n, 256b + i] of a GGUF Q6_K matrix in float64 (exact)."""
    rec = _k_records(buf, n_rows, k, _Q6_K_RECORD, Q6_K_BLOCK_BYTES)
    nb = k // QK_K
    d = rec["d"].astype(np.float64)                             # [n][nb]
    scales = rec["scales"].astype(np.float64)                   # [n][nb][16]
    ql = rec["ql"].astype(np.int64).reshape(n_rows, nb, 2, 64)  # half t
    qh = rec["qh"].astype(np.int64).reshape(n_rows, nb, 2, 32)
    q = np.empty((n_rows, nb, 2, 4, 32), dtype=np.int64)        # half t, k, l
    for kk in range(4):
        nib = ql[..., 32 * (kk % 2):32 * (kk % 2) + 32]
        low = (nib & 0x0F) if kk < 2 else (nib >> 4)
        high = (qh >> (2 * kk)) & 3
        q[:, :, :, kk, :] = low | (high << 4)
    q = q.reshape(n_rows, nb, QK_K)                             # weight 128t + 32k + l
    s = np.repeat(scales, 16, axis=2)                           # scale of weight i: i // 16
    w = d[:, :, None] * s * (q - 32)
    return w.reshape(n_rows, -1)


def q4_k_linear_ref(w_q4k, n: int, k: int, x) -> np.ndarray:
    """y = x . W^T for a GGUF Q4_K weight W [n][k] (float64)."""
    return np.asarray(x, dtype=np.float64) @ dequantize_q4_k(w_q4k, n, k).T


def q5_k_linear_ref(w_q5k, n: int, k: int, x) -> np.ndarray:
    """y = x . W^T for a GGUF Q5_K weight W [n][k] (float64)."""
    return np.asarray(x, dtype=np.float64) @ dequantize_q5_k(w_q5k, n, k).T


def q6_k_linear_ref(w_q6k, n: int, k: int, x) -> np.ndarray:
    """y = x . W^T for a GGUF Q6_K weight W [n][k] (float64)."""
    return np.asarray(x, dtype=np.float64) @ dequantize_q6_k(w_q6k, n, k).T


def fused_gate_up_silu_q4_k_ref(w, f: int, k: int, x) -> np.ndarray:
    """SiLU(x . W_gate^T) * (x . W_up^T) from one Q4_K [2f][k] matrix, gate rows first."""
    y = q4_k_linear_ref(w, 2 * f, k, x)
    return silu_ref(y[:, :f]) * y[:, f:]


def fused_gate_up_silu_q5_k_ref(w, f: int, k: int, x) -> np.ndarray:
    """SiLU(x . W_gate^T) * (x . W_up^T) from one Q5_K [2f][k] matrix, gate rows first."""
    yy = q5_k_linear_ref(w, 2 * f, k, x)
    return silu_ref(yy[:, :f]) * yy[:, f:]


def fused_gate_up_silu_q6_k_ref(w, f: int, k: int, x) -> np.ndarray:
    """SiLU(x . W_gate^T) * (x . W_up^T) from one Q6_K [2f][k] matrix, gate rows first."""
    y = q6_k_linear_ref(w, 2 * f, k, x)
    return silu_ref(y[:, :f]) * y[:, f:]


# ------------------------------------------------------------------------- linear


def q8_linear_ref(w_q8, n: int, k: int, x) -> np.ndarray:
    """y = x . W^T for a Q8_0 weight W [n][k] and activation rows x [M][k].

    The packed-weight linear of section 14.1 (LinearWeight), written as the plain
    definition: dequantize, then one float64 matrix product.
    """
    x64 = np.asarray(x, dtype=np.float64)
    if x64.ndim != 2 or x64.shape[1] != k:
        raise ValueError(f"x must be [M][{k}], got {x64.shape}")
    w = dequantize_q8_0(w_q8, n, k)
    return x64 @ w.T


def sigmoid_ref(g) -> np.ndarray:
    """Logistic function in the overflow-free form for both signs of g."""
    g = np.asarray(g, dtype=np.float64)
    out = np.empty_like(g)
    pos = g >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-g[pos]))
    e = np.exp(g[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def silu_ref(g) -> np.ndarray:
    """SiLU(g) = g * sigmoid(g) (the activation of the SwiGLU FFN, section 14.2)."""
    g = np.asarray(g, dtype=np.float64)
    return g * sigmoid_ref(g)


def fused_gate_up_silu_ref(w_gate_up_q8, f: int, k: int, x) -> np.ndarray:
    """h = SiLU(x . W_gate^T) * (x . W_up^T) from one fused gate_up matrix [2f][k].

    Section 14.1 fuses gate and up into one gate_up matrix; section 14.2 gives the
    SwiGLU FFN.  Gate rows are [0, f), up rows are [f, 2f).
    """
    y = q8_linear_ref(w_gate_up_q8, 2 * f, k, x)
    g = y[:, :f]
    u = y[:, f:]
    return silu_ref(g) * u


# ------------------------------------------------------------------------- router


def router_logits_ref(x, w_router) -> np.ndarray:
    """logits[m, e] = x[m] . w_router[e] in float64."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w_router, dtype=np.float64).T


def softmax_ref(logits) -> np.ndarray:
    """Row softmax with the row maximum subtracted first."""
    l = np.asarray(logits, dtype=np.float64)
    z = l - l.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def route_topk_ref(x, w_router, k: int, normalize: bool = True):
    """Softmax top-k routing (section 14.2: routerTopK, normalize_selected = norm_topk_prob).

    p = softmax(x . W_r^T); the k experts of largest p are chosen, in descending
    order of p with ties to the lower expert index (a stable sort of -p); the chosen
    weights are p[sel], divided by their sum when ``normalize``.

    Returns (idx int32 [M][k], w float64 [M][k]).
    """
    logits = router_logits_ref(x, w_router)
    m_rows, n_exp = logits.shape
    if not 1 <= k <= n_exp:
        raise ValueError(f"k={k} must be in [1, {n_exp}]")
    p = softmax_ref(logits)
    idx = np.empty((m_rows, k), dtype=np.int32)
    wts = np.empty((m_rows, k), dtype=np.float64)
    for m in range(m_rows):
        order = np.argsort(-p[m], kind="stable")
        sel = order[:k]
        idx[m] = sel
        chosen = p[m, sel]
        wts[m] = chosen / chosen.sum() if normalize else chosen
    return idx, wts


def route_topk_p_ref(x, w_router, k: int, normalize: bool = True, top_p: float = 1.0):
    """Softmax top-k routing followed by adaptive expert top-p (section 14.2 Config:
    moe_expert_top_p, 1.0 = full top-k; applyExpertTopP).

    The pages give the knob and its neutral value only; the reading taken here (parity
    pinned by hand values, the p = 1 identity and brute force, not by a page's numbers):
    with the chosen probabilities p_0 >= p_1 >= ... >= p_{k-1} (the top-k of the softmax,
    in selection order) and c_j = (p_0 + ... + p_j) / (p_0 + ... + p_{k-1}), slot 0 is
    always kept and slot j >= 1 is kept while c_{j-1} < top_p; top_p >= 1 keeps all k.
    Kept weights are p_j, divided by the kept sum when ``normalize``; a dropped slot gets
    expert index -1 and weight 0.

    Returns (idx int32 [M][k], w float64 [M][k]).
    """
    logits = router_logits_ref(x, w_router)
    m_rows, n_exp = logits.shape
    if not 1 <= k <= n_exp:
        raise ValueError(f"k={k} must be in [1, {n_exp}]")
    if not 0.0 < top_p <= 1.0:
        raise ValueError("top_p must be in (0, 1]")
    p = softmax_ref(logits)
    idx = np.full((m_rows, k), -1, dtype=np.int32)
    wts = np.zeros((m_rows, k), dtype=np.float64)
    for m in range(m_rows):
        sel = np.argsort(-p[m], kind="stable")[:k]
        chosen = p[m, sel]
        total = chosen.sum()
        kept = 1
        while kept < k and (top_p >= 1.0 or chosen[:kept].sum() / total < top_p):
            kept += 1
        idx[m, :kept] = sel[:kept]
        wts[m, :kept] = chosen[:kept] / chosen[:kept].sum() if normalize else chosen[:kept]
    return idx, wts


# ---------------------------------------------------------------------------- MoE


def _expert_slice(stack, e: int, rows: int, k: int):
    """Bytes of expert e in a Q8_0 expert stack laid out [E][rows][k]."""
    raw = np.frombuffer(memoryview(stack).cast("B"), dtype=np.uint8)
    nb = rows * q8_0_row_bytes(k)
    return raw[e * nb:(e + 1) * nb]


def moe_mixture_ref(w_gate_up_exps, w_down_exps, n_exp: int, f: int, h: int,
                    x, topk_idx, topk_w) -> np.ndarray:
    """Router-weighted SwiGLU mixture for given routing (section 14.2: moeSwiGluFfnSeq).

    y[m] = sum_j topk_w[m, j] * W_down[e] . (SiLU(W_gate[e] x_m) * (W_up[e] x_m)),
    e = topk_idx[m, j], summed over slots j = 0 .. k-1 in order (section 14.4 keeps
    each token's summation order fixed).  Expert stacks are Q8_0 [E][2f][h] (gate_up)
    and [E][h][f] (down).  An index of -1 marks a slot that expert top-p dropped: it
    contributes nothing.
    """
    x64 = np.asarray(x, dtype=np.float64)
    idx = np.asarray(topk_idx)
    wts = np.asarray(topk_w, dtype=np.float64)
    m_rows, k_used = idx.shape
    y = np.zeros((m_rows, h), dtype=np.float64)
    for m in range(m_rows):
        for j in range(k_used):
            e = int(idx[m, j])
            if e == -1:
                continue
            if not 0 <= e < n_exp:
                raise ValueError(f"expert index {e} out of range [0, {n_exp})")
            hid = fused_gate_up_silu_ref(_expert_slice(w_gate_up_exps, e, 2 * f, h), f, h,
                                         x64[m:m + 1])
            out = q8_linear_ref(_expert_slice(w_down_exps, e, h, f), h, f, hid)
            y[m] += wts[m, j] * out[0]
    return y


def moe_ref(w_router, w_gate_up_exps, w_down_exps, n_exp: int, f: int, h: int,
            x, k: int, normalize: bool = True):
    """Route (softmax top-k), then the mixture.  Returns (y, idx, w)."""
    idx, wts = route_topk_ref(x, w_router, k, normalize)
    y = moe_mixture_ref(w_gate_up_exps, w_down_exps, n_exp, f, h, x, idx, wts)
    return y, idx, wts


# ------------------------------------------------------- diagnostic (not a gate)


def bf16_round_ref(a) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as float64.

    Goes through float32 first; each value here is already a float32 (activations,
    or fp32(d)*q), so that step is exact.
    """
    a32 = np.asarray(a, dtype=np.float32)
    bits = a32.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    return rounded.astype(np.uint32).view(np.float32).astype(np.float64)


def q8_linear_bf16_operands_ref(w_q8, n: int, k: int, x) -> np.ndarray:
    """Diagnostic: y with both operands rounded to bfloat16 first, float64 sums.

    Isolates the accumulation error of a bf16 matrix-core path from its operand
    rounding.  Not a parity gate.
    """
    w = dequantize_q8_0(w_q8, n, k)
    return bf16_round_ref(np.asarray(x, dtype=np.float32)) @ bf16_round_ref(w).T


# ---------------------------------- integer q8 x q8 path (quantized activations)
#
# The DGX Spark README (Features; Architecture) names GEMV kernels that read Q8_0
# directly through int8 dot products (dp4a), and the qwen3 runner README (the q8_0
# KV cache example; the --cache-type flag) names an integer q8 x q8 dot path over
# quantized blocks.  No page defines the activation code; the reading taken here
# (pinned by hand values, properties and exact identities, not by a page's numbers):
# per block of 32 inputs, amax = max |x|; the scale is dx = amax / 127 and the codes
# are q = round-half-even(x * (127 / amax)), both quotients and the product rounded
# to float32, so that the integer codes are decided in float32 exactly as on the
# device.  A block with amax below 2^-120 (all zeros included) gets dx = 0, q = 0:
# there 127 / amax would leave the float32 range.  Inputs are finite.

ACT_ZERO_BELOW = np.float32(2.0 ** -120)   # smaller block maxima are coded as zero


def quantize_act_q8_ref(x):
    """Per-32-input int8 codes and float32 scales of float32 activation rows.

    Returns (q int8 [m][k], dx float32 [m][k/32]); |q| <= 127.
    """
    x32 = np.asarray(x, dtype=np.float32)
    m, k = x32.shape
    if k % QK8_0:
        raise ValueError("k must be a multiple of 32")
    blocks = x32.reshape(m, k // QK8_0, QK8_0)
    amax = np.max(np.abs(blocks), axis=2)
    nz = amax >= ACT_ZERO_BELOW
    safe = np.where(nz, amax, np.float32(1)).astype(np.float32)
    inv = np.where(nz, np.float32(127) / safe, np.float32(0)).astype(np.float32)
    dx = np.where(nz, safe / np.float32(127), np.float32(0)).astype(np.float32)
    prod = (blocks * inv[:, :, None]).astype(np.float32)
    q = np.clip(np.rint(prod), -127, 127).astype(np.int8)
    return q.reshape(m, k), dx


def q8_linear_codes_ref(w_q8, n: int, k: int, qx, dx) -> np.ndarray:
    """y[m, n] = sum_b d_w[n, b] * dx[m, b] * (sum_i q_w[n, b, i] * q_x[m, b, i]).

    qx: int8 codes [m][k] (any int8 value), dx: float32 scales [m][k/32].  The block
    dot products are exact integers (int64); the scaling and the sum over blocks run in
    float64.
    """
    dw, qwf = parse_q8_0(w_q8, n, k)                      # [n][nb], [n][nb][32]
    qw = qwf.astype(np.int64)                             # exact: the quants are integers
    qx = np.asarray(qx, dtype=np.int64)
    dx = np.asarray(dx, dtype=np.float32).astype(np.float64)
    m = qx.shape[0]
    qx = qx.reshape(m, k // QK8_0, QK8_0)
    out = np.empty((m, n), dtype=np.float64)
    for mi in range(m):
        isum = np.einsum("nbi,bi->nb", qw, qx[mi])       # exact integer block dots
        out[mi] = (dw * dx[mi][None, :] * isum).sum(axis=1)
    return out


def q8_linear_q8act_ref(w_q8, n: int, k: int, x) -> np.ndarray:
    """The linear on activations quantized by quantize_act_q8_ref."""
    qx, dx = quantize_act_q8_ref(x)
    return q8_linear_codes_ref(w_q8, n, k, qx, dx)


def fused_gate_up_silu_codes_ref(w_gate_up_q8, f: int, k: int, qx, dx) -> np.ndarray:
    """SiLU(gate) * up with both products on the given codes (gate rows [0, f))."""
    y = q8_linear_codes_ref(w_gate_up_q8, 2 * f, k, qx, dx)
    return silu_ref(y[:, :f]) * y[:, f:]


def fused_gate_up_silu_q8act_ref(w_gate_up_q8, f: int, k: int, x) -> np.ndarray:
    """SiLU(gate) * up on activations quantized by quantize_act_q8_ref."""
    qx, dx = quantize_act_q8_ref(x)
    return fused_gate_up_silu_codes_ref(w_gate_up_q8, f, k, qx, dx)


# ----------------------------------------------------------- error measurement


def rel_err_row_norm(y, y_ref) -> float:
    """max over rows of max|y - y_ref| / ||y_ref row||_2 (0 when the row is all zero)."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(y_ref, dtype=np.float64)
    if y.shape != r.shape:
        raise ValueError(f"shape mismatch {y.shape} vs {r.shape}")
    if y.size == 0:
        return 0.0
    y2 = y.reshape(-1, y.shape[-1])
    r2 = r.reshape(-1, r.shape[-1])
    worst = 0.0
    for a, b in zip(y2, r2):
        nrm = math.sqrt(float(np.dot(b, b)))
        d = float(np.max(np.abs(a - b)))
        if nrm == 0.0:
            if d != 0.0:
                return math.inf
            continue
        worst = max(worst, d / nrm)
    return worst


def rel_err_row_max(y, y_ref) -> float:
    """max over rows of max|y - y_ref| / max|y_ref row| (the stricter reading)."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(y_ref, dtype=np.float64)
    if y.size == 0:
        return 0.0
    y2 = y.reshape(-1, y.shape[-1])
    r2 = r.reshape(-1, r.shape[-1])
    worst = 0.0
    for a, b in zip(y2, r2):
        mx = float(np.max(np.abs(b)))
        d = float(np.max(np.abs(a - b)))
        if mx == 0.0:
            if d != 0.0:
                return math.inf
            continue
        worst = max(worst, d / mx)
    return worst
