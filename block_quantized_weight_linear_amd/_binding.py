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
for _name in ("q4_k_linear", "q4_k_linear_fused_gate_up_silu", "q5_k_linear", "q5_k_linear_fused_gate_up_silu",
              "q6_k_linear", "q6_k_linear_fused_gate_up_silu"):
    getattr(lib, _name).restype = ctypes.c_int
    getattr(lib, _name).argtypes = [_vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp]
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

lib.q8_moe_grouped_linear_noalloc.restype = ctypes.c_int
lib.q8_moe_grouped_linear_noalloc.argtypes = [_vp, _vp, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _i32, _vp,
                                              _i64, _vp]

# measurement aids (include/q8_probe.h)
lib.q8_probe_shape_count.restype = _i32
lib.q8_probe_shape_count.argtypes = []
lib.q8_probe_sink_words.restype = _i64
lib.q8_probe_sink_words.argtypes = [_i32]
lib.q8_probe_stream_read.restype = ctypes.c_int
lib.q8_probe_stream_read.argtypes = [_vp, _i64, _i32, _vp, _i64, _vp]
lib.q8_probe_empty.restype = ctypes.c_int
lib.q8_probe_empty.argtypes = [_i64, _vp]

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


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t, dtype, name, device=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _ld(x, width):
    """Leading dimension to pass for a 2-D tensor whose rows hold `width` used values."""
    if x.shape[0] <= 1:  # a single row: only its first `width` values are touched
        return width + (-width % 4)
    return x.stride(0)


def _rows_in(x, width, name):
    """A 2-D [m][width] input with unit column stride and rows that do not overlap."""
    if x.dim() != 2 or x.shape[1] != width:
        raise ValueError(f"{name} must be [m][{width}], got {tuple(x.shape)}")
    if x.numel() and (x.stride(1) != 1 or (x.shape[0] > 1 and x.stride(0) < width)):
        raise ValueError(f"{name} must have contiguous, non-overlapping rows")
    return x.shape[0]


def _rows_out(out, m, width, name, dtype, device):
    """A caller-supplied output: exactly [m][width], unit column stride, rows that do not
    overlap (the kernels write m rows of width values at the tensor's row stride)."""
    _dev(out, dtype, name, device)
    if out.dim() != 2 or tuple(out.shape) != (m, width):
        raise ValueError(f"{name} must be [{m}][{width}], got {tuple(out.shape)}")
    if out.numel() and (out.stride(1) != 1 or (m > 1 and out.stride(0) < width)):
        raise ValueError(f"{name} must have unit column stride and non-overlapping rows")
    return out


def _contig_out(t, shape, name, dtype, device):
    _dev(t, dtype, name, device)
    if tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {list(shape)} tensor, got {tuple(t.shape)}")
    return t


def _bytes(w, need, name, device):
    """A byte tensor (uint8, contiguous) holding at least `need` bytes."""
    _dev(w, torch.uint8, name, device)
    if not w.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if w.numel() < need:
        raise ValueError(f"{name} holds {w.numel()} bytes, the shape needs {need}")
    return w


# bytes per 256 weights of each packed format
Q8_0_BYTES, Q4_0_BYTES, Q4_K_BYTES, Q5_K_BYTES, Q6_K_BYTES = 272, 144, 144, 176, 210


def _quant_bytes(rows, k, bytes_256):
    if k <= 0 or k % 256 or rows < 0:
        return 0  # the library reports the shape error
    return rows * (k // 256) * bytes_256


def _call(device, fn, *args):
    # the library launches on the current device: make it the tensors' device
    with torch.cuda.device(device):
        check(fn(*args))


def _dense(fn, w, n_w, n_out, k, x, out, bytes_256):
    """Shared marshalling of the dense linears: weight rows n_w, outputs n_out."""
    _dev(x, torch.float32, "x")
    dev = x.device
    m = _rows_in(x, k, "x")
    _bytes(w, _quant_bytes(n_w, k, bytes_256) if n_out and m else 0, "w", dev)
    if out is None:
        out = torch.empty((m, n_out), dtype=torch.float32, device=dev)
    _rows_out(out, m, n_out, "out", torch.float32, dev)
    _call(dev, fn, w.data_ptr(), n_out, k, x.data_ptr(), m, _ld(x, k), out.data_ptr(), _ld(out, n_out),
          _stream(x))
    return out


def q8_linear(w, n: int, k: int, x, out=None):
    """y = x . W^T for a Q8_0 weight W [n][k] (uint8 bytes) and float32 x [m][k]."""
    return _dense(lib.q8_linear, w, n, n, k, x, out, Q8_0_BYTES)


def q8_linear_fused_gate_up_silu(w, f: int, k: int, x, out=None):
    """h = SiLU(x . W_gate^T) * (x . W_up^T); W is Q8_0 [2f][k], gate rows first."""
    return _dense(lib.q8_linear_fused_gate_up_silu, w, 2 * f, f, k, x, out, Q8_0_BYTES)


def q4_0_linear(w, n: int, k: int, x, out=None):
    """y = x . W^T for a GGUF Q4_0 weight W [n][k] (uint8 bytes) and float32 x [m][k]."""
    return _dense(lib.q4_0_linear, w, n, n, k, x, out, Q4_0_BYTES)


def q4_0_linear_fused_gate_up_silu(w, f: int, k: int, x, out=None):
    """h = SiLU(x . W_gate^T) * (x . W_up^T); W is GGUF Q4_0 [2f][k], gate rows first."""
    return _dense(lib.q4_0_linear_fused_gate_up_silu, w, 2 * f, f, k, x, out, Q4_0_BYTES)


def q4_k_linear(w, n: int, k: int, x, out=None):
    """y = x . W^T for a GGUF Q4_K weight W [n][k] (uint8 bytes) and float32 x [m][k]."""
    return _dense(lib.q4_k_linear, w, n, n, k, x, out, Q4_K_BYTES)


def q4_k_linear_fused_gate_up_silu(w, f: int, k: int, x, out=None):
    """h = SiLU(x . W_gate^T) * (x . W_up^T); W is GGUF Q4_K [2f][k], gate rows first."""
    return _dense(lib.q4_k_linear_fused_gate_up_silu, w, 2 * f, f, k, x, out, Q4_K_BYTES)


def q5_k_linear(w, n: int, k: int, x, out=None):
    """y = x . W^T for a GGUF Q5_K weight W [n][k] (uint8 bytes) and float32 x [m][k]."""
    return _dense(lib.q5_k_linear, w, n, n, k, x, out, Q5_K_BYTES)


def q5_k_linear_fused_gate_up_silu(w, f: int, k: int, x, out=None):
    """h = SiLU(x . W_gate^T) * (x . W_up^T); W is GGUF Q5_K [2f][k], gate rows first."""
    return _dense(lib.q5_k_linear_fused_gate_up_silu, w, 2 * f, f, k, x, out, Q5_K_BYTES)


def q6_k_linear(w, n: int, k: int, x, out=None):
    """y = x . W^T for a GGUF Q6_K weight W [n][k] (uint8 bytes) and float32 x [m][k]."""
    return _dense(lib.q6_k_linear, w, n, n, k, x, out, Q6_K_BYTES)


def q6_k_linear_fused_gate_up_silu(w, f: int, k: int, x, out=None):
    """h = SiLU(x . W_gate^T) * (x . W_up^T); W is GGUF Q6_K [2f][k], gate rows first."""
    return _dense(lib.q6_k_linear_fused_gate_up_silu, w, 2 * f, f, k, x, out, Q6_K_BYTES)


def q8_quantize_act(x, xq=None, xd=None):
    """Int8 codes [m][k] and float32 scales [m][k/32] of float32 activation rows x [m][k]."""
    _dev(x, torch.float32, "x")
    if x.dim() != 2:
        raise ValueError("x must be [m][k]")
    m, k = x.shape
    _rows_in(x, k, "x")
    dev = x.device
    if xq is None:
        xq = torch.empty((m, k), dtype=torch.int8, device=dev)
    if xd is None:
        xd = torch.empty((m, k // 32), dtype=torch.float32, device=dev)
    _contig_out(xq, (m, k), "xq", torch.int8, dev)
    _contig_out(xd, (m, k // 32), "xd", torch.float32, dev)
    _call(dev, lib.q8_quantize_act, x.data_ptr(), m, k, _ld(x, k), xq.data_ptr(), xd.data_ptr(), _stream(x))
    return xq, xd


def _codes(xq, xd, k):
    _dev(xq, torch.int8, "xq")
    _dev(xd, torch.float32, "xd", xq.device)
    if xq.dim() != 2 or xq.shape[1] != k or not xq.is_contiguous():
        raise ValueError(f"xq must be a contiguous [m][{k}] tensor")
    m = xq.shape[0]
    if tuple(xd.shape) != (m, k // 32) or not xd.is_contiguous():
        raise ValueError(f"xd must be a contiguous [m][{k // 32}] tensor")
    return m


def _dense_codes(fn, w, n_w, n_out, k, xq, xd, out):
    m = _codes(xq, xd, k)
    dev = xq.device
    _bytes(w, _quant_bytes(n_w, k, Q8_0_BYTES) if n_out and m else 0, "w", dev)
    if out is None:
        out = torch.empty((m, n_out), dtype=torch.float32, device=dev)
    _rows_out(out, m, n_out, "out", torch.float32, dev)
    _call(dev, fn, w.data_ptr(), n_out, k, xq.data_ptr(), xd.data_ptr(), m, out.data_ptr(), _ld(out, n_out),
          _stream(xq))
    return out


def q8_linear_q8act(w, n: int, k: int, xq, xd, out=None):
    """y = the Q8_0 weight W [n][k] against int8 activation codes xq [m][k] with scales xd."""
    return _dense_codes(lib.q8_linear_q8act, w, n, n, k, xq, xd, out)


def q8_linear_fused_gate_up_silu_q8act(w, f: int, k: int, xq, xd, out=None):
    """h = SiLU(gate) * up from a fused Q8_0 gate_up matrix [2f][k] on int8 activation codes."""
    return _dense_codes(lib.q8_linear_fused_gate_up_silu_q8act, w, 2 * f, f, k, xq, xd, out)


def moe_route_topk(x, w_router, k: int, normalize: bool = True, idx_out=None, w_out=None, top_p=None,
                   workspace=None):
    """Softmax top-k routing; returns (topk_idx int32 [m][k], topk_w float32 [m][k]).

    With top_p (in (0, 1]) the adaptive expert top-p cut follows (moe_route_topk_top_p):
    dropped slots hold expert -1 and weight 0.  With a workspace (uint8 device tensor of
    at least moe_route_workspace_bytes(m, n_exp) bytes; True allocates one) the two-pass
    form runs (moe_route_topk_ws), bit-identical to the one-pass calls."""
    _dev(x, torch.float32, "x")
    dev = x.device
    _dev(w_router, torch.float32, "w_router", dev)
    if not w_router.is_contiguous() or w_router.dim() != 2:
        raise ValueError("w_router must be a contiguous [n_exp][h] tensor")
    n_exp, h = w_router.shape
    m = _rows_in(x, h, "x")
    if idx_out is None:
        idx_out = torch.empty((m, k), dtype=torch.int32, device=dev)
    if w_out is None:
        w_out = torch.empty((m, k), dtype=torch.float32, device=dev)
    _contig_out(idx_out, (m, k), "idx_out", torch.int32, dev)
    _contig_out(w_out, (m, k), "w_out", torch.float32, dev)
    norm = 1 if normalize else 0
    if workspace is not None:
        if workspace is True:
            workspace = torch.empty(max(moe_route_workspace_bytes(m, n_exp), 1), dtype=torch.uint8, device=dev)
        _bytes(workspace, 0, "workspace", dev)
        _call(dev, lib.moe_route_topk_ws, x.data_ptr(), m, h, _ld(x, h), w_router.data_ptr(), n_exp, k, norm,
              1.0 if top_p is None else float(top_p), idx_out.data_ptr(), w_out.data_ptr(), workspace.data_ptr(),
              workspace.numel(), _stream(x))
    elif top_p is None:
        _call(dev, lib.moe_route_topk, x.data_ptr(), m, h, _ld(x, h), w_router.data_ptr(), n_exp, k, norm,
              idx_out.data_ptr(), w_out.data_ptr(), _stream(x))
    else:
        _call(dev, lib.moe_route_topk_top_p, x.data_ptr(), m, h, _ld(x, h), w_router.data_ptr(), n_exp, k, norm,
              float(top_p), idx_out.data_ptr(), w_out.data_ptr(), _stream(x))
    return idx_out, w_out


def moe_route_workspace_bytes(m: int, n_exp: int) -> int:
    return int(lib.moe_route_workspace_bytes(m, n_exp))


def q8_moe_workspace_bytes(m: int, k: int, n_exp: int, f: int, h: int) -> int:
    return int(lib.q8_moe_workspace_bytes(m, k, n_exp, f, h))


def _moe_args(w_gate_up_exps, w_down_exps, n_exp, f, h, x, topk_idx, topk_w, out):
    _dev(x, torch.float32, "x")
    dev = x.device
    m = _rows_in(x, h, "x")
    _dev(topk_idx, torch.int32, "topk_idx", dev)
    _dev(topk_w, torch.float32, "topk_w", dev)
    if topk_idx.dim() != 2 or topk_idx.shape[0] != m or not topk_idx.is_contiguous():
        raise ValueError("topk_idx must be a contiguous [m][k] tensor")
    k = topk_idx.shape[1]
    _contig_out(topk_w, (m, k), "topk_w", torch.float32, dev)
    _bytes(w_gate_up_exps, _quant_bytes(n_exp * 2 * f, h, Q8_0_BYTES) if m else 0, "w_gate_up_exps", dev)
    _bytes(w_down_exps, _quant_bytes(n_exp * h, f, Q8_0_BYTES) if m else 0, "w_down_exps", dev)
    if out is None:
        out = torch.empty((m, h), dtype=torch.float32, device=dev)
    _rows_out(out, m, h, "out", torch.float32, dev)
    return dev, m, k, out


def q8_moe_grouped_linear(w_gate_up_exps, w_down_exps, n_exp: int, f: int, h: int, x, topk_idx, topk_w,
                          out=None, workspace=None):
    """Router-weighted SwiGLU expert mixture; returns y float32 [m][h]."""
    dev, m, k, out = _moe_args(w_gate_up_exps, w_down_exps, n_exp, f, h, x, topk_idx, topk_w, out)
    need = q8_moe_workspace_bytes(m, k, n_exp, f, h) if m else 0
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _bytes(workspace, 0, "workspace", dev)
    _call(dev, lib.q8_moe_grouped_linear, w_gate_up_exps.data_ptr(), w_down_exps.data_ptr(), n_exp, f, h,
          x.data_ptr(), m, _ld(x, h), topk_idx.data_ptr(), topk_w.data_ptr(), k, out.data_ptr(), _ld(out, h),
          workspace.data_ptr(), workspace.numel(), _stream(x))
    return out


def q8_moe_grouped_linear_noalloc(w_gate_up_exps, w_down_exps, n_exp: int, f: int, h: int, x, topk_idx, topk_w,
                                  out=None):
    """The same mixture with the library's fixed per-device scratch instead of a workspace
    (the C entry point allocates nothing; pass `out` to keep this wrapper allocation-free
    too).  Sizes whose workspace exceeds the scratch raise Q8Error."""
    dev, m, k, out = _moe_args(w_gate_up_exps, w_down_exps, n_exp, f, h, x, topk_idx, topk_w, out)
    _call(dev, lib.q8_moe_grouped_linear_noalloc, w_gate_up_exps.data_ptr(), w_down_exps.data_ptr(), n_exp, f, h,
          x.data_ptr(), m, _ld(x, h), topk_idx.data_ptr(), topk_w.data_ptr(), k, out.data_ptr(), _ld(out, h),
          _stream(x))
    return out


# ------------------------------------------------------------ measurement aids


def probe_shape_count() -> int:
    """Launch shapes of probe_stream_read (0 .. count-1)."""
    return int(lib.q8_probe_shape_count())


def probe_stream_read(buf, nbytes: int, shape: int, sink=None):
    """Plain streaming read of the first nbytes bytes of a device byte tensor in one
    launch (launch shape `shape`), for a benchmark's read ceiling; returns the sink
    tensor of per-lane xor words."""
    _bytes(buf, nbytes, "buf", None)
    with torch.cuda.device(buf.device):
        words = int(lib.q8_probe_sink_words(shape))
    if words < 0:
        raise ValueError(f"probe shape {shape} is out of range [0, {probe_shape_count()})")
    if sink is None:
        sink = torch.empty(words, dtype=torch.int32, device=buf.device)
    _contig_out(sink, (words,), "sink", torch.int32, buf.device)
    _call(buf.device, lib.q8_probe_stream_read, buf.data_ptr(), nbytes, shape, sink.data_ptr(), words, _stream(buf))
    return sink


def probe_empty(blocks: int, device=None):
    """One launch of `blocks` workgroups that do nothing, on the current stream."""
    device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    with torch.cuda.device(device):
        check(lib.q8_probe_empty(blocks, ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)))
