"""The C ABI library on the host (no GPU needed): it loads, exports every function the
header declares, and rejects bad arguments before touching the device.

None of these calls reaches a kernel: every argument error is detected on the host,
and zero-size calls return before any HIP call.
"""

from __future__ import annotations

import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

q8 = pytest.importorskip("block_quantized_weight_linear_amd")
lib = q8.lib

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_WORKSPACE, ERR_DEVICE = range(6)
FAKE = 0x10000  # 64 KiB: a 256-byte aligned, non-null address that is never dereferenced


def declared_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("q8_linear", "q8_linear_fused_gate_up_silu", "moe_route_topk", "q8_moe_grouped_linear",
              "q8_moe_workspace_bytes", "q8_status_string", "q8_last_error", "q8_abi_version",
              "q8_quantize_act", "q8_linear_q8act", "q8_linear_fused_gate_up_silu_q8act",
              "moe_route_topk_top_p", "moe_route_topk_ws", "moe_route_workspace_bytes",
              "q4_0_linear", "q4_0_linear_fused_gate_up_silu", "q8_moe_grouped_linear_noalloc",
              "q4_k_linear", "q4_k_linear_fused_gate_up_silu", "q6_k_linear", "q6_k_linear_fused_gate_up_silu",
              "q5_k_linear", "q5_k_linear_fused_gate_up_silu", "q8_probe_stream_read", "q8_probe_empty",
              "q8_probe_shape_count", "q8_probe_sink_words"):
        assert n in names, names


def test_library_exports_every_declared_symbol():
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert q8.abi_version() == 8


def test_status_strings():
    for s in range(6):
        assert lib.q8_status_string(s)
    assert lib.q8_status_string(99) == b"unknown status"


LINEAR_FORMATS = {"q8_0": ("q8_linear", "q8_linear_fused_gate_up_silu"),
                  "q4_0": ("q4_0_linear", "q4_0_linear_fused_gate_up_silu"),
                  "q4_k": ("q4_k_linear", "q4_k_linear_fused_gate_up_silu"),
                  "q5_k": ("q5_k_linear", "q5_k_linear_fused_gate_up_silu"),
                  "q6_k": ("q6_k_linear", "q6_k_linear_fused_gate_up_silu")}


def _lin_base(w=FAKE, n=64, k=256, x=FAKE, m=1, ldx=256, y=FAKE, ldy=64, fused=False, q4="q8_0"):
    fn = getattr(lib, LINEAR_FORMATS[q4][1 if fused else 0])
    return fn(w, n, k, x, m, ldx, y, ldy, None)


@pytest.mark.parametrize("q4", sorted(LINEAR_FORMATS))
@pytest.mark.parametrize("fused", [False, True])
def test_linear_argument_errors(fused, q4):
    def _lin(**kw):
        return _lin_base(q4=q4, **kw)

    assert _lin(k=0, fused=fused) == ERR_SHAPE
    assert _lin(k=32, fused=fused) == ERR_SHAPE          # a Q8_0 multiple but not of 256
    assert _lin(k=384, fused=fused) == ERR_SHAPE
    assert _lin(n=-1, fused=fused) == ERR_SHAPE
    assert _lin(m=-3, fused=fused) == ERR_SHAPE
    assert _lin(ldx=128, fused=fused) == ERR_SHAPE
    assert _lin(ldy=63, fused=fused) == ERR_SHAPE
    assert _lin(w=None, fused=fused) == ERR_NULL
    assert _lin(x=None, fused=fused) == ERR_NULL
    assert _lin(y=None, fused=fused) == ERR_NULL
    assert _lin(w=FAKE + 4, fused=fused) == ERR_ALIGN
    assert _lin(x=FAKE + 8, fused=fused) == ERR_ALIGN
    assert _lin(m=2, ldx=258, fused=fused) == ERR_ALIGN
    assert _lin(y=FAKE + 2, fused=fused) == ERR_ALIGN
    msg = lib.q8_last_error().decode()
    assert "aligned" in msg


_lin = _lin_base


def _lin8(w=FAKE, n=64, k=256, xq=FAKE, xd=FAKE, m=1, y=FAKE, ldy=64, fused=False):
    fn = lib.q8_linear_fused_gate_up_silu_q8act if fused else lib.q8_linear_q8act
    return fn(w, n, k, xq, xd, m, y, ldy, None)


@pytest.mark.parametrize("fused", [False, True])
def test_q8act_linear_argument_errors(fused):
    assert _lin8(fused=fused, k=0) == ERR_SHAPE
    assert _lin8(fused=fused, k=320) == ERR_SHAPE
    assert _lin8(fused=fused, n=-1) == ERR_SHAPE
    assert _lin8(fused=fused, m=-1) == ERR_SHAPE
    assert _lin8(fused=fused, ldy=63) == ERR_SHAPE
    assert _lin8(fused=fused, xq=None) == ERR_NULL
    assert _lin8(fused=fused, xd=None) == ERR_NULL
    assert _lin8(fused=fused, w=None) == ERR_NULL
    assert _lin8(fused=fused, xq=FAKE + 8) == ERR_ALIGN
    assert _lin8(fused=fused, xd=FAKE + 4) == ERR_ALIGN
    assert _lin8(fused=fused, w=FAKE + 4) == ERR_ALIGN
    assert _lin8(fused=fused, y=FAKE + 1) == ERR_ALIGN
    assert _lin8(fused=fused, m=0, w=None, xq=None, xd=None, y=None) == OK
    assert _lin8(fused=fused, n=0, ldy=0, w=None, xq=None, xd=None, y=None) == OK


def test_quantize_act_argument_errors():
    def call(x=FAKE, m=2, k=256, ldx=256, xq=FAKE, xd=FAKE):
        return lib.q8_quantize_act(x, m, k, ldx, xq, xd, None)

    assert call(k=96) == ERR_SHAPE
    assert call(m=-1) == ERR_SHAPE
    assert call(ldx=255) == ERR_SHAPE
    assert call(x=None) == ERR_NULL
    assert call(xq=None) == ERR_NULL
    assert call(xd=None) == ERR_NULL
    assert call(x=FAKE + 4) == ERR_ALIGN
    assert call(xq=FAKE + 4) == ERR_ALIGN
    assert call(ldx=258) == ERR_ALIGN
    assert call(m=0, x=None, xq=None, xd=None) == OK
    assert "q8_quantize_act" in lib.q8_last_error().decode() or lib.q8_last_error() == b""


def test_zero_sizes_enqueue_nothing():
    # no rows or no outputs: valid, nothing enqueued, pointers may be null
    assert _lin(m=0, w=None, x=None, y=None) == OK
    assert _lin(n=0, w=None, x=None, y=None, ldy=0) == OK
    assert lib.moe_route_topk(None, 0, 256, 256, None, 8, 2, 1, None, None, None) == OK
    assert lib.q8_moe_grouped_linear(None, None, 8, 256, 256, None, 0, 256, None, None, 2, None, 256,
                                     None, 0, None) == OK


def test_route_argument_errors():
    def call(x=FAKE, m=2, h=256, ldx=256, w=FAKE, e=8, k=2, idx=FAKE, wt=FAKE):
        return lib.moe_route_topk(x, m, h, ldx, w, e, k, 1, idx, wt, None)

    assert call(h=100) == ERR_SHAPE
    assert call(e=0) == ERR_SHAPE
    assert call(e=257) == ERR_SHAPE
    assert call(k=0) == ERR_SHAPE
    assert call(k=9) == ERR_SHAPE
    assert call(ldx=128) == ERR_SHAPE
    assert call(x=None) == ERR_NULL
    assert call(idx=None) == ERR_NULL
    assert call(w=FAKE + 4) == ERR_ALIGN
    assert call(wt=FAKE + 2) == ERR_ALIGN


def test_route_top_p_argument_errors():
    def call(top_p, x=FAKE, m=2, k=2):
        return lib.moe_route_topk_top_p(x, m, 256, 256, FAKE, 8, k, 1, ctypes.c_float(top_p), FAKE, FAKE, None)

    assert call(0.0) == ERR_SHAPE
    assert call(-0.5) == ERR_SHAPE
    assert call(1.5) == ERR_SHAPE
    assert call(float("nan")) == ERR_SHAPE
    assert "top_p" in lib.q8_last_error().decode()
    assert call(0.5, k=9) == ERR_SHAPE
    assert call(0.5, x=None) == ERR_NULL
    assert call(0.5, m=0, x=None) == OK


def test_route_ws_argument_errors():
    need = lib.moe_route_workspace_bytes(16, 128)
    assert need >= 16 * 128 * 4 and need % 256 == 0
    assert lib.moe_route_workspace_bytes(16, 0) == 0
    assert lib.moe_route_workspace_bytes(-1, 8) == 0

    def call(ws=FAKE, wsb=None, m=2, top_p=1.0, x=FAKE):
        if wsb is None:
            wsb = lib.moe_route_workspace_bytes(m, 8)
        return lib.moe_route_topk_ws(x, m, 256, 256, FAKE, 8, 2, 1, ctypes.c_float(top_p), FAKE, FAKE, ws, wsb, None)

    assert call(ws=None) == ERR_WORKSPACE
    assert call(wsb=8) == ERR_WORKSPACE
    assert call(ws=FAKE + 4) == ERR_ALIGN
    assert call(top_p=0.0) == ERR_SHAPE
    assert call(x=None) == ERR_NULL
    assert call(m=0, x=None, ws=None) == OK


def test_moe_workspace_and_errors():
    need = lib.q8_moe_workspace_bytes(16, 8, 128, 768, 2048)
    pairs = 16 * 8
    assert need >= 4 * (129 + 2 * pairs) + 4 * pairs * (768 + 2048)
    assert need % 256 == 0
    assert lib.q8_moe_workspace_bytes(16, 9, 8, 768, 2048) == 0      # k > n_exp
    assert lib.q8_moe_workspace_bytes(16, 2, 8, 100, 2048) == 0      # f not a multiple of 256
    assert lib.q8_moe_workspace_bytes(16, 2, 8, 768, 32768) == 0     # h above 16384

    def call(e=8, f=256, h=256, m=2, k=2, ws=FAKE, wsb=None, idx=FAKE):
        if wsb is None:
            wsb = lib.q8_moe_workspace_bytes(m, k, e, f, h)
        return lib.q8_moe_grouped_linear(FAKE, FAKE, e, f, h, FAKE, m, 256, idx, FAKE, k, FAKE, 256, ws, wsb, None)

    assert call(wsb=16) == ERR_WORKSPACE
    assert call(ws=None) == ERR_WORKSPACE
    assert call(ws=FAKE + 16) == ERR_ALIGN
    assert call(k=9) == ERR_SHAPE
    assert call(f=200) == ERR_SHAPE
    assert call(idx=None) == ERR_NULL


def test_error_text_is_thread_local():
    import threading

    assert _lin(k=32) == ERR_SHAPE
    here = lib.q8_last_error().decode()
    seen = {}

    def other():
        seen["t"] = lib.q8_last_error().decode()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert "k=32" in here and seen["t"] == ""


def test_one_hip_runtime_in_process():
    """torch bundles a HIP runtime with the same soname as the one the library links;
    the binding imports torch first so only one copy is ever mapped."""
    maps = open("/proc/self/maps").read()
    paths = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(paths) == 1, paths


def test_moe_noalloc_refuses_sizes_beyond_its_scratch():
    """The no-allocation mixture refuses, on the host, sizes whose workspace exceeds its
    fixed 16 MiB scratch (nothing is enqueued); argument errors are reported as for the
    workspace form; zero rows is a valid no-op."""
    scratch = 16 << 20
    # A3B sizes: 146 tokens x 8 slots fit, 147 do not
    assert lib.q8_moe_workspace_bytes(146, 8, 128, 768, 2048) <= scratch
    assert lib.q8_moe_workspace_bytes(147, 8, 128, 768, 2048) > scratch

    def call(m, k=8, e=128, f=768, h=2048, idx=FAKE):
        return lib.q8_moe_grouped_linear_noalloc(FAKE, FAKE, e, f, h, FAKE, m, h, idx, FAKE, k, FAKE, h, None)

    assert call(147) == ERR_WORKSPACE
    assert "scratch" in lib.q8_last_error().decode()
    assert call(2048) == ERR_WORKSPACE
    assert call(4, k=129) == ERR_SHAPE
    assert call(4, f=700) == ERR_SHAPE
    assert call(4, idx=None) == ERR_NULL
    assert call(0, idx=None) == OK


def test_probe_argument_errors():
    """The measurement aids reject bad arguments on the host (no launch)."""
    f = lib.q8_probe_stream_read
    assert lib.q8_probe_shape_count() >= 1
    assert lib.q8_probe_sink_words(-1) == -1
    assert lib.q8_probe_sink_words(lib.q8_probe_shape_count()) == -1
    assert f(None, 4096, 0, FAKE, 1 << 20, None) == ERR_NULL
    assert f(FAKE, 4096, 0, None, 1 << 20, None) == ERR_NULL
    assert f(FAKE, 0, 0, FAKE, 1 << 20, None) == ERR_SHAPE
    assert f(FAKE, 4000, 0, FAKE, 1 << 20, None) == ERR_SHAPE
    assert f(FAKE, 4096, -1, FAKE, 1 << 20, None) == ERR_SHAPE
    assert f(FAKE, 4096, lib.q8_probe_shape_count(), FAKE, 1 << 20, None) == ERR_SHAPE
    assert f(FAKE + 8, 4096, 0, FAKE, 1 << 20, None) == ERR_ALIGN
    assert f(FAKE, 4096, 0, FAKE + 2, 1 << 20, None) == ERR_ALIGN
    assert b"probe" in lib.q8_last_error()
    assert lib.q8_probe_empty(0, None) == ERR_SHAPE
    assert lib.q8_probe_empty(1 << 31, None) == ERR_SHAPE
