"""ctypes binding of include/q8_linear.h.

Argument marshalling only: checks tensor dtypes/devices, allocates outputs with
torch when none are given, passes raw device pointers, sizes and torch's current
HIP stream, and turns a non-zero status into Q8Error.  Every step of the
computation runs in the HIP library; there is no fallback.  Importing raises if
the library has not been built.
"""

from __future__ import annotations

import ctypes
import os

# torch ships its own HIP runtime (libamdhip64.so.7).  The library links the same
# soname, and the first copy loaded serves the whole process; importing torch first
# makes that torch's copy, so tensors, streams and our kernels share one runtime.
import torch  # noqa: F401  (imported for its side effect on the loaded HIP runtime)

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libq8linear.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: the HIP library has not been built "
        "(python -m block_quantized_weight_linear_amd.build)")

lib = ctypes.CDLL(LIB_PATH)

_i64, _i32, _vp, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t

lib.q8_abi_version.restype = _i32
lib.q8_abi_version.argtypes = []
lib.q8_status_string.restype = ctypes.c_char_p
lib.q8_status_string.argtypes = [ctypes.c_int]
lib.q8_last_error.restype = ctypes.c_char_p
lib.q8_last_error.argtypes = []
lib.q8_linear.restype = ctypes.c_int
lib.q8_linear.argtypes = [_vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp]
lib.q8_linear_fused_gate_up_silu.restype = ctypes.c_int
lib.q8_linear_fused_gate_up_silu.argtypes = [_vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp]
lib.q4_0_linear.restype = ctypes.c_int
lib.q4_0_linear.argtypes = [_vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp]
lib.q4_0_linear_fused_gate_up_silu.restype = ctypes.c_int
lib.q4_0_linear_fused_gate_up_silu.argtypes = [_vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp]
lib.q8_quantize_act.restype = ctypes.c_int
lib.q8_quantize_act.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _vp]
lib.q8_linear_q8act.restype = ctypes.c_int
lib.q8_linear_q8act.argtypes = [_vp, _i64, _i64, _vp, _vp, _i64, _vp, _i64, _vp]
lib.q8_linear_fused_gate_up_silu_q8act.restype = ctypes.c_int
lib.q8_linear_fused_gate_up_silu_q8act.argtypes = [_vp, _i64, _i64, _vp, _vp, _i64, _vp, _i64, _vp]
lib.moe_route_topk.restype = ctypes.c_int
lib.moe_route_topk.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _i32, _i32, _vp, _vp, _vp]
lib.moe_route_topk_top_p.restype = ctypes.c_int
lib.moe_route_topk_top_p.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _i32, _i32, ctypes.c_float, _vp, _vp, _vp]
lib.moe_route_workspace_bytes.restype = _sz
lib.moe_route_workspace_bytes.argtypes = [_i64, _i64]
lib.moe_route_topk_ws.restype = ctypes.c_int
lib.moe_route_topk_ws.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _i32, _i32, ctypes.c_float, _vp, _vp, _vp, _sz,
                                  _vp]
lib.q8_moe_workspace_bytes.restype = _sz
lib.q8_moe_workspace_bytes.argtypes = [_i64, _i32, _i64, _i64, _i64]
lib.q8_moe_grouped_linear.restype = ctypes.c_int
lib.q8_moe_grouped_linear.argtypes = [_vp, _vp, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _i32, _vp, _i64,
                                      _vp, _sz, _vp]

Q8_OK, Q8_ERR_NULL, Q8_ERR_SHAPE, Q8_ERR_ALIGN, Q8_ERR_WORKSPACE, Q8_ERR_DEVICE = range(6)


class Q8Error(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{lib.q8_status_string(status).decode()} ({status}): {detail}")


def check(status: int) -> None:
    if status != Q8_OK:
        raise Q8Error(status, lib.q8_last_error().decode())


def abi_version() -> int:
    return int(lib.q8_abi_version())


def _torch():
    return torch


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t, dtype, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _ld(x, width):
    """Leading dimension to pass for a 2-D tensor whose rows hold `width` used values."""
    if x.shape[0] <= 1:  # a single row: only its first `width` values are touched
        return width + (-width % 4)
    return x.stride(0)


def q8_linear(w, n: int, k: int, x, out=None):
    """y = x . W^T for a Q8_0 weight W [n][k] (uint8 bytes) and float32 x [m][k]."""
    torch = _torch()
    _dev(w, torch.uint8, "w")
    _dev(x, torch.float32, "x")
    if x.dim() != 2 or x.shape[1] != k or (x.numel() and x.stride(1) != 1):
        raise ValueError(f"x must be [m][{k}] with contiguous rows")
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _dev(out, torch.float32, "out")
    check(lib.q8_linear(w.data_ptr(), n, k, x.data_ptr(), m, _ld(x, k), out.data_ptr(), _ld(out, n), _stream(x)))
    return out


def q8_linear_fused_gate_up_silu(w, f: int, k: int, x, out=None):
    """h = SiLU(x . W_gate^T) * (x . W_up^T); W is Q8_0 [2f][k], gate rows first."""
    torch = _torch()
    _dev(w, torch.uint8, "w")
    _dev(x, torch.float32, "x")
    if x.dim() != 2 or x.shape[1] != k or (x.numel() and x.stride(1) != 1):
        raise ValueError(f"x must be [m][{k}] with contiguous rows")
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, f), dtype=torch.float32, device=x.device)
    _dev(out, torch.float32, "out")
    check(lib.q8_linear_fused_gate_up_silu(w.data_ptr(), f, k, x.data_ptr(), m, _ld(x, k), out.data_ptr(),
                                           _ld(out, f), _stream(x)))
    return out


def q4_0_linear(w, n: int, k: int, x, out=None):
    """y = x . W^T for a GGUF Q4_0 weight W [n][k] (uint8 bytes) and float32 x [m][k]."""
    torch = _torch()
    _dev(w, torch.uint8, "w")
    _dev(x, torch.float32, "x")
    if x.dim() != 2 or x.shape[1] != k or (x.numel() and x.stride(1) != 1):
        raise ValueError(f"x must be [m][{k}] with contiguous rows")
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _dev(out, torch.float32, "out")
    check(lib.q4_0_linear(w.data_ptr(), n, k, x.data_ptr(), m, _ld(x, k), out.data_ptr(), _ld(out, n), _stream(x)))
    return out


def q4_0_linear_fused_gate_up_silu(w, f: int, k: int, x, out=None):
    """h = SiLU(x . W_gate^T) * (x . W_up^T); W is GGUF Q4_0 [2f][k], gate rows first."""
    torch = _torch()
    _dev(w, torch.uint8, "w")
    _dev(x, torch.float32, "x")
    if x.dim() != 2 or x.shape[1] != k or (x.numel() and x.stride(1) != 1):
        raise ValueError(f"x must be [m][{k}] with contiguous rows")
    m = x.shape[0]
    if out is None:
        out = torch.empty((m, f), dtype=torch.float32, device=x.device)
    _dev(out, torch.float32, "out")
    check(lib.q4_0_linear_fused_gate_up_silu(w.data_ptr(), f, k, x.data_ptr(), m, _ld(x, k), out.data_ptr(),
                                             _ld(out, f), _stream(x)))
    return out


def q8_quantize_act(x, xq=None, xd=None):
    """Int8 codes [m][k] and float32 scales [m][k/32] of float32 activation rows x [m][k]."""
    torch = _torch()
    _dev(x, torch.float32, "x")
    if x.dim() != 2 or (x.numel() and x.stride(1) != 1):
        raise ValueError("x must be [m][k] with contiguous rows")
    m, k = x.shape
    if xq is None:
        xq = torch.empty((m, k), dtype=torch.int8, device=x.device)
    if xd is None:
        xd = torch.empty((m, k // 32), dtype=torch.float32, device=x.device)
    _dev(xq, torch.int8, "xq")
    _dev(xd, torch.float32, "xd")
    if tuple(xq.shape) != (m, k) or tuple(xd.shape) != (m, k // 32) or not (xq.is_contiguous() and xd.is_contiguous()):
        raise ValueError("xq must be a contiguous [m][k] tensor and xd a contiguous [m][k/32] tensor")
    check(lib.q8_quantize_act(x.data_ptr(), m, k, _ld(x, k), xq.data_ptr(), xd.data_ptr(), _stream(x)))
    return xq, xd


def _codes(xq, xd, k):
    torch = _torch()
    _dev(xq, torch.int8, "xq")
    _dev(xd, torch.float32, "xd")
    if xq.dim() != 2 or xq.shape[1] != k or not xq.is_contiguous():
        raise ValueError(f"xq must be a contiguous [m][{k}] tensor")
    m = xq.shape[0]
    if tuple(xd.shape) != (m, k // 32) or not xd.is_contiguous():
        raise ValueError(f"xd must be a contiguous [m][{k // 32}] tensor")
    return m


def q8_linear_q8act(w, n: int, k: int, xq, xd, out=None):
    """y = the Q8_0 weight W [n][k] against int8 activation codes xq [m][k] with scales xd."""
    torch = _torch()
    _dev(w, torch.uint8, "w")
    m = _codes(xq, xd, k)
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=xq.device)
    _dev(out, torch.float32, "out")
    check(lib.q8_linear_q8act(w.data_ptr(), n, k, xq.data_ptr(), xd.data_ptr(), m, out.data_ptr(), _ld(out, n),
                              _stream(xq)))
    return out


def q8_linear_fused_gate_up_silu_q8act(w, f: int, k: int, xq, xd, out=None):
    """h = SiLU(gate) * up from a fused Q8_0 gate_up matrix [2f][k] on int8 activation codes."""
    torch = _torch()
    _dev(w, torch.uint8, "w")
    m = _codes(xq, xd, k)
    if out is None:
        out = torch.empty((m, f), dtype=torch.float32, device=xq.device)
    _dev(out, torch.float32, "out")
    check(lib.q8_linear_fused_gate_up_silu_q8act(w.data_ptr(), f, k, xq.data_ptr(), xd.data_ptr(), m,
                                                 out.data_ptr(), _ld(out, f), _stream(xq)))
    return out


def moe_route_topk(x, w_router, k: int, normalize: bool = True, idx_out=None, w_out=None, top_p=None,
                   workspace=None):
    """Softmax top-k routing; returns (topk_idx int32 [m][k], topk_w float32 [m][k]).

    With top_p (in (0, 1]) the adaptive expert top-p cut follows (moe_route_topk_top_p):
    dropped slots hold expert -1 and weight 0.  With a workspace (uint8 device tensor of
    at least moe_route_workspace_bytes(m, n_exp) bytes; True allocates one) the two-pass
    form runs (moe_route_topk_ws), bit-identical to the one-pass calls."""
    torch = _torch()
    _dev(x, torch.float32, "x")
    _dev(w_router, torch.float32, "w_router")
    if not w_router.is_contiguous() or w_router.dim() != 2:
        raise ValueError("w_router must be a contiguous [n_exp][h] tensor")
    n_exp, h = w_router.shape
    if x.dim() != 2 or x.shape[1] != h or (x.numel() and x.stride(1) != 1):
        raise ValueError(f"x must be [m][{h}] with contiguous rows")
    m = x.shape[0]
    if idx_out is None:
        idx_out = torch.empty((m, k), dtype=torch.int32, device=x.device)
    if w_out is None:
        w_out = torch.empty((m, k), dtype=torch.float32, device=x.device)
    _dev(idx_out, torch.int32, "idx_out")
    _dev(w_out, torch.float32, "w_out")
    if not (idx_out.is_contiguous() and w_out.is_contiguous()):
        raise ValueError("idx_out and w_out must be contiguous")
    if workspace is not None:
        if workspace is True:
            workspace = torch.empty(max(moe_route_workspace_bytes(m, n_exp), 1), dtype=torch.uint8,
                                    device=x.device)
        _dev(workspace, torch.uint8, "workspace")
        check(lib.moe_route_topk_ws(x.data_ptr(), m, h, _ld(x, h), w_router.data_ptr(), n_exp, k,
                                    1 if normalize else 0, 1.0 if top_p is None else float(top_p),
                                    idx_out.data_ptr(), w_out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                    _stream(x)))
    elif top_p is None:
        check(lib.moe_route_topk(x.data_ptr(), m, h, _ld(x, h), w_router.data_ptr(), n_exp, k,
                                 1 if normalize else 0, idx_out.data_ptr(), w_out.data_ptr(), _stream(x)))
    else:
        check(lib.moe_route_topk_top_p(x.data_ptr(), m, h, _ld(x, h), w_router.data_ptr(), n_exp, k,
                                       1 if normalize else 0, float(top_p), idx_out.data_ptr(), w_out.data_ptr(),
                                       _stream(x)))
    return idx_out, w_out


def moe_route_workspace_bytes(m: int, n_exp: int) -> int:
    return int(lib.moe_route_workspace_bytes(m, n_exp))


def q8_moe_workspace_bytes(m: int, k: int, n_exp: int, f: int, h: int) -> int:
    return int(lib.q8_moe_workspace_bytes(m, k, n_exp, f, h))


def q8_moe_grouped_linear(w_gate_up_exps, w_down_exps, n_exp: int, f: int, h: int, x, topk_idx, topk_w,
                          out=None, workspace=None):
    """Router-weighted SwiGLU expert mixture; returns y float32 [m][h]."""
    torch = _torch()
    _dev(w_gate_up_exps, torch.uint8, "w_gate_up_exps")
    _dev(w_down_exps, torch.uint8, "w_down_exps")
    _dev(x, torch.float32, "x")
    _dev(topk_idx, torch.int32, "topk_idx")
    _dev(topk_w, torch.float32, "topk_w")
    if x.dim() != 2 or x.shape[1] != h or (x.numel() and x.stride(1) != 1):
        raise ValueError(f"x must be [m][{h}] with contiguous rows")
    m = x.shape[0]
    if topk_idx.dim() != 2 or topk_idx.shape[0] != m or not topk_idx.is_contiguous():
        raise ValueError("topk_idx must be a contiguous [m][k] tensor")
    k = topk_idx.shape[1]
    if tuple(topk_w.shape) != (m, k) or not topk_w.is_contiguous():
        raise ValueError("topk_w must be a contiguous [m][k] tensor")
    if out is None:
        out = torch.empty((m, h), dtype=torch.float32, device=x.device)
    _dev(out, torch.float32, "out")
    need = q8_moe_workspace_bytes(m, k, n_exp, f, h) if m else 0
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _dev(workspace, torch.uint8, "workspace")
    check(lib.q8_moe_grouped_linear(w_gate_up_exps.data_ptr(), w_down_exps.data_ptr(), n_exp, f, h, x.data_ptr(), m,
                                    _ld(x, h), topk_idx.data_ptr(), topk_w.data_ptr(), k, out.data_ptr(),
                                    _ld(out, h), workspace.data_ptr(), workspace.numel(), _stream(x)))
    return out
