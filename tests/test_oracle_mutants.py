"""Plant plausible mistakes in copies of the oracle (on the CPU) and require that the
pins in test_oracle_pins.py catch each one.  This shows the pins are strong enough
that a dropped term, a wrong sign, index or byte order, or a transposed operand in
the oracle cannot pass unnoticed.
"""

from __future__ import annotations

import os
import types

import pytest

import test_oracle_pins as pins

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "q8_oracle.py")

MUTANTS = {
    "scale_big_endian": ('("d", "<f2"), ("qs", "i1"', '("d", ">f2"), ("qs", "i1"'),
    "q4_0_scale_big_endian": ('("d", "<f2"), ("qs", "u1"', '("d", ">f2"), ("qs", "u1"'),
    "quants_unsigned": ('("qs", "i1", (QK8_0,))', '("qs", "u1", (QK8_0,))'),
    "dropped_scale": ("w = d[:, :, None] * q", "w = q + 0 * d[:, :, None]"),
    "reversed_k": ("return w.reshape(n_rows, k)", "return w.reshape(n_rows, k)[:, ::-1]"),
    "gate_up_swapped": ("g = y[:, :f]\n    u = y[:, f:]", "g = y[:, f:]\n    u = y[:, :f]"),
    "silu_sign": ("return g * sigmoid_ref(g)", "return g * sigmoid_ref(-g)"),
    "sigmoid_negative_branch": ("out[~pos] = e / (1.0 + e)", "out[~pos] = 1.0 / (1.0 + e)"),
    "ties_to_higher_index": ('order = np.argsort(-p[m], kind="stable")', "order = np.argsort(p[m], kind=\"stable\")[::-1]"),
    "no_renormalize": ("wts[m] = chosen / chosen.sum() if normalize else chosen", "wts[m] = chosen"),
    "softmax_wrong_axis": ("return e / e.sum(axis=-1, keepdims=True)", "return e / e.sum(axis=0, keepdims=True)"),
    "moe_ignores_weights": ("y[m] += wts[m, j] * out[0]", "y[m] += out[0]"),
    "moe_wrong_expert": ("return raw[e * nb:(e + 1) * nb]", "return raw[(e ^ 1) * nb:((e ^ 1) + 1) * nb]"),
    "router_untransposed_logits": ("@ np.asarray(w_router, dtype=np.float64).T",
                                   "@ np.asarray(w_router, dtype=np.float64).T[::-1].T"),
    "top_p_cut_inclusive": ("chosen[:kept].sum() / total < top_p", "chosen[:kept].sum() / total <= top_p"),
    "top_p_full_softmax_cumulative": ("chosen[:kept].sum() / total < top_p", "chosen[:kept].sum() < top_p"),
    "top_p_normalize_by_topk_total": ("chosen[:kept] / chosen[:kept].sum() if normalize", "chosen[:kept] / total if normalize"),
    "top_p_ignores_knob": ("kept = 1\n", "kept = k\n"),
    "q4_0_nibbles_interleaved": ("q[:, :, :16] = qs & 0x0F\n    q[:, :, 16:] = qs >> 4",
                                 "q[:, :, 0::2] = qs & 0x0F\n    q[:, :, 1::2] = qs >> 4"),
    "q4_0_nibbles_swapped": ("q[:, :, :16] = qs & 0x0F\n    q[:, :, 16:] = qs >> 4",
                             "q[:, :, :16] = qs >> 4\n    q[:, :, 16:] = qs & 0x0F"),
    "q4_0_no_offset": ("(d[:, :, None] * (q - 8.0))", "(d[:, :, None] * q)"),
    "q4_0_signed_nibbles": ("(d[:, :, None] * (q - 8.0))", "(d[:, :, None] * np.where(q > 7, q - 16.0, q))"),
    "act_round_floor": ("q = np.clip(np.rint(prod), -127, 127)", "q = np.clip(np.floor(prod), -127, 127)"),
    "act_round_half_away": ("q = np.clip(np.rint(prod), -127, 127)",
                            "q = np.clip(np.trunc(prod + np.copysign(np.float32(0.5), prod)), -127, 127)"),
    "act_scale_inverted": ("dx = np.where(nz, safe / np.float32(127), np.float32(0))",
                           "dx = np.where(nz, np.float32(127) / safe, np.float32(0))"),
    "act_amax_signed": ("amax = np.max(np.abs(blocks), axis=2)", "amax = np.max(blocks, axis=2)"),
    "q8act_drops_dx": ("(dw * dx[mi][None, :] * isum)", "(dw * isum)"),
    "act_zero_only_exact_zero": ("nz = amax >= ACT_ZERO_BELOW", "nz = amax > 0"),
    "q4_k_scale_min_swapped": ("sc[..., j] = b[..., j] & 63\n        m[..., j] = b[..., j + 4] & 63",
                               "sc[..., j] = b[..., j + 4] & 63\n        m[..., j] = b[..., j] & 63"),
    "q4_k_top_bits_from_scale_byte": ("m[..., j] = (b[..., j + 4] >> 4) | ((b[..., j] >> 6) << 4)",
                                      "m[..., j] = (b[..., j + 4] >> 4) | ((b[..., j - 4] >> 6) << 4)"),
    "q4_k_high_bits_unshifted": ("sc[..., j] = (b[..., j + 4] & 0x0F) | ((b[..., j - 4] >> 6) << 4)",
                                 "sc[..., j] = (b[..., j + 4] & 0x0F) | (b[..., j - 4] >> 6)"),
    "q4_k_nibbles_swapped": ("q[:, :, :, 0, :] = qs & 0x0F\n    q[:, :, :, 1, :] = qs >> 4",
                             "q[:, :, :, 0, :] = qs >> 4\n    q[:, :, :, 1, :] = qs & 0x0F"),
    "q4_k_min_added": ("* q - (dmin[:, :, None, None]", "* q + (dmin[:, :, None, None]"),
    "q4_k_d_dmin_swapped": ('_Q4_K_RECORD = np.dtype([("d", "<f2"), ("dmin", "<f2")',
                            '_Q4_K_RECORD = np.dtype([("dmin", "<f2"), ("d", "<f2")'),
    "q6_k_qh_shift": ("high = (qh >> (2 * kk)) & 3", "high = (qh >> kk) & 3"),
    "q6_k_no_offset": ("w = d[:, :, None] * s * (q - 32)", "w = d[:, :, None] * s * q"),
    "q6_k_scale_per_32": ("s = np.repeat(scales, 16, axis=2)", "s = np.repeat(scales[:, :, :8], 32, axis=2)"),
    "q6_k_ql_half_offset": ("nib = ql[..., 32 * (kk % 2):32 * (kk % 2) + 32]", "nib = ql[..., 32 * (kk // 2):32 * (kk // 2) + 32]"),
    "q6_k_nibble_choice": ("low = (nib & 0x0F) if kk < 2 else (nib >> 4)", "low = (nib & 0x0F) if kk % 2 == 0 else (nib >> 4)"),
    "q6_k_scales_unsigned": ('("scales", "i1", (QK_K // 16,))', '("scales", "u1", (QK_K // 16,))'),
    "q5_k_top_bit_index": ("top = (qh >> (2 * c + half)) & 1", "top = (qh >> (c + half)) & 1"),
    "q5_k_top_bit_weight": ("q5[:, :, c, half, :] = low4 + 16 * top", "q5[:, :, c, half, :] = low4 + 32 * top"),
    "q5_k_nibble_order": ("low4 = (qs[:, :, c, :] >> (4 * half)) & 0x0F", "low4 = (qs[:, :, c, :] >> (4 - 4 * half)) & 0x0F"),
    "q5_k_qh_after_quants": ('("scales", "u1", (12,)), ("qh", "u1", (QK_K // 8,)),\n                         ("qs", "u1", (QK_K // 2,))',
                             '("scales", "u1", (12,)), ("qs", "u1", (QK_K // 2,)),\n                         ("qh", "u1", (QK_K // 8,))'),
    "q5_k_min_added": ("* q5 - (dmin[:, :, None, None]", "* q5 + (dmin[:, :, None, None]"),
    "q8act_wrong_block": ('isum = np.einsum("nbi,bi->nb", qw, qx[mi])', 'isum = np.einsum("nbi,bi->nb", qw, qx[mi][::-1])'),
}


def _mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC_PATH).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/absent"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src.replace(old, new), SRC_PATH, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    mod = _mutant(name)
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check(mod)
        except Exception:  # an assertion or a crash both count as caught
            caught.append(check.__name__)
    assert caught, f"no pin caught mutant {name}"
