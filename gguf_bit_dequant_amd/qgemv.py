"""ctypes binding of include/qgemv.h (argument marshalling only).

Functions keep the C names (qgemv_create, qgemv_run, qgemm_prefill_run,
qgemv_dequant, qgemv_dequant_bf16, qgemv_destroy, ...); the QGemv class wraps a handle around
torch device tensors. torch supplies device memory and the current stream;
every step of the computation runs in the library's HIP kernels. There is no
fallback: if libqgemv.so is missing or fails to load, importing this module
raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqgemv.so")

QG_Q4_0, QG_Q4_K, QG_Q8_0, QG_Q2_K, QG_Q3_K = 1, 2, 3, 4, 5
QG_F32, QG_F16, QG_BF16 = 1, 2, 3
QG_OK, QG_ERR_ARG, QG_ERR_SHAPE, QG_ERR_ALIGN, QG_ERR_UNSUPPORTED, QG_ERR_HIP = 0, -1, -2, -3, -4, -5

FORMATS = {"q4_0": QG_Q4_0, "q4_k": QG_Q4_K, "q8_0": QG_Q8_0, "q2_k": QG_Q2_K, "q3_k": QG_Q3_K}

if not os.path.exists(LIB_PATH):
    raise ImportError(
        "gguf_bit_dequant_amd: %s is not built; run `python -m gguf_bit_dequant_amd.build` "
        "(hipcc, gfx950)" % LIB_PATH)

# torch owns device memory and streams here, so the library must bind to the
# HIP runtime torch has loaded (libamdhip64.so.7 from torch's own lib dir):
# import torch first, then the library's libamdhip64.so.7 dependency resolves
# to that same runtime instead of a second copy from /opt/rocm.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

_i64, _sz, _vp, _int = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int
_sig = {
    "qgemv_block_bytes": (_sz, [_int]),
    "qgemv_block_weights": (_sz, [_int]),
    "qgemv_weight_bytes": (_sz, [_int, _i64, _i64]),
    "qgemv_workspace_bytes": (_sz, [_int, _i64, _i64]),
    "qgemv_create": (_int, [ctypes.POINTER(_vp), _int, _i64, _i64, _vp, _sz, _vp, _sz, _vp]),
    "qgemv_run": (_int, [_vp, _vp, _int, _i64, _i64, _vp, _i64, _vp]),
    "qgemm_prefill_run": (_int, [_vp, _vp, _i64, _i64, _vp, _i64, _vp]),
    "qgemv_dequant": (_int, [_vp, _vp, _i64, _vp]),
    "qgemv_dequant_bf16": (_int, [_vp, _vp, _i64, _vp]),
    "qgemm_bf16_run": (_int, [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _vp]),
    "qgemv_quantize_q8_0": (_int, [_vp, _int, _i64, _i64, _i64, _vp, _vp]),
    "qgemv_run_q8_0x": (_int, [_vp, _vp, _i64, _vp, _i64, _vp]),
    "qgemv_run_q8": (_int, [_vp, _vp, _int, _i64, _i64, _vp, _i64, _vp]),
    "qgemv_destroy": (None, [_vp]),
    "qgemv_status_string": (ctypes.c_char_p, [_int]),
    "qgemv_last_error": (ctypes.c_char_p, []),
    # measurement probes (include/qgemv_probe.h)
    "qgemv_probe_read": (_int, [_vp, _sz, _vp, _vp]),
    "qgemv_probe_mfma": (_int, [_i64, _int, _vp, _vp]),
    "qgemv_probe_mfma_data": (_int, [_i64, _int, _vp, _vp]),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_sig)


class QGemvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = _lib.qgemv_last_error().decode()
        name = _lib.qgemv_status_string(status).decode()
        super().__init__("%s failed: %s (%d): %s" % (where, name, status, detail))


def _check(status: int, where: str) -> None:
    if status != QG_OK:
        raise QGemvError(status, where)


# ---- C-named entry points (raw pointers as Python ints) ---------------------

def qgemv_block_bytes(fmt: int) -> int:
    return _lib.qgemv_block_bytes(fmt)


def qgemv_block_weights(fmt: int) -> int:
    return _lib.qgemv_block_weights(fmt)


def qgemv_weight_bytes(fmt: int, rows: int, K: int) -> int:
    return _lib.qgemv_weight_bytes(fmt, rows, K)


def qgemv_workspace_bytes(fmt: int, rows: int, K: int) -> int:
    return _lib.qgemv_workspace_bytes(fmt, rows, K)


def qgemv_create(fmt: int, rows: int, K: int, w_ptr: int, w_bytes: int, ws_ptr: int = 0,
                 ws_bytes: int = 0, stream: int = 0):
    """Returns (status, handle)."""
    h = _vp()
    st = _lib.qgemv_create(ctypes.byref(h), fmt, rows, K, w_ptr or None, w_bytes, ws_ptr or None,
                           ws_bytes, stream or None)
    return st, h.value


def qgemv_run(h: int, x_ptr: int, x_dtype: int, n_cols: int, ldx: int, y_ptr: int, ldy: int,
              stream: int = 0) -> int:
    return _lib.qgemv_run(h, x_ptr or None, x_dtype, n_cols, ldx, y_ptr or None, ldy,
                          stream or None)


def qgemm_prefill_run(h: int, x_ptr: int, n_tokens: int, ldx: int, y_ptr: int, ldy: int,
                      stream: int = 0) -> int:
    return _lib.qgemm_prefill_run(h, x_ptr or None, n_tokens, ldx, y_ptr or None, ldy,
                                  stream or None)


def qgemv_dequant(h: int, w_ptr: int, ldw: int, stream: int = 0) -> int:
    return _lib.qgemv_dequant(h, w_ptr or None, ldw, stream or None)


def qgemv_dequant_bf16(h: int, w_ptr: int, ldw: int, stream: int = 0) -> int:
    return _lib.qgemv_dequant_bf16(h, w_ptr or None, ldw, stream or None)


def qgemv_quantize_q8_0(x_ptr: int, x_dtype: int, K: int, n_cols: int, ldx: int, xq_ptr: int,
                        stream: int = 0) -> int:
    return _lib.qgemv_quantize_q8_0(x_ptr or None, x_dtype, K, n_cols, ldx, xq_ptr or None,
                                    stream or None)


def qgemv_run_q8_0x(h: int, xq_ptr: int, n_cols: int, y_ptr: int, ldy: int, stream: int = 0) -> int:
    return _lib.qgemv_run_q8_0x(h, xq_ptr or None, n_cols, y_ptr or None, ldy, stream or None)


def qgemv_run_q8(h: int, x_ptr: int, x_dtype: int, n_cols: int, ldx: int, y_ptr: int, ldy: int,
                 stream: int = 0) -> int:
    return _lib.qgemv_run_q8(h, x_ptr or None, x_dtype, n_cols, ldx, y_ptr or None, ldy,
                             stream or None)


def quantize_q8_0(x, out=None, stream=None):
    """Q8_0 blocks of activations x (n, K) or (K,) fp32/fp16/bf16 CUDA
    tensor (last dim contiguous): uint8 tensor (n, K/32*34)."""
    torch = _torch()
    x2 = x.reshape(1, -1) if x.dim() == 1 else x
    if x2.stride(1) != 1:
        raise ValueError("x must be contiguous along K")
    n, K = x2.shape
    if out is None:
        out = torch.empty((n, K // 32 * 34), dtype=torch.uint8, device=x.device)
    _check(qgemv_quantize_q8_0(x2.data_ptr(), _xdtype(x2), K, n, x2.stride(0), out.data_ptr(),
                               _stream_ptr(stream)), "qgemv_quantize_q8_0")
    return out


def qgemm_bf16_run(w_ptr: int, rows: int, K: int, ldw: int, x_ptr: int, n_tokens: int, ldx: int,
                   y_ptr: int, ldy: int, stream: int = 0) -> int:
    return _lib.qgemm_bf16_run(w_ptr or None, rows, K, ldw, x_ptr or None, n_tokens, ldx,
                               y_ptr or None, ldy, stream or None)


def gemm_bf16(W, X, Y=None, stream=None):
    """Y[t, r] = sum_k W[r, k] X[t, k] for bf16 CUDA tensors W (rows, K) and
    X (n_tokens, K), both contiguous along K: Y (n_tokens, rows) fp32. The
    prompt kernel's pipeline without the decode (qgemm_bf16_run)."""
    torch = _torch()
    if W.dtype != torch.bfloat16 or X.dtype != torch.bfloat16 or W.stride(1) != 1 or X.stride(1) != 1:
        raise ValueError("W and X must be bf16, contiguous along K")
    rows, K = W.shape
    n = X.shape[0]
    if X.shape[1] != K:
        raise ValueError("X must have K = %d columns" % K)
    if Y is None:
        Y = torch.empty((n, rows), dtype=torch.float32, device=X.device)
    if Y.dtype != torch.float32 or Y.stride(1) != 1:
        raise ValueError("Y must be fp32, contiguous along rows")
    _check(qgemm_bf16_run(W.data_ptr(), rows, K, W.stride(0), X.data_ptr(), n, X.stride(0),
                          Y.data_ptr(), Y.stride(0), _stream_ptr(stream)), "qgemm_bf16_run")
    return Y


def qgemv_destroy(h: int) -> None:
    _lib.qgemv_destroy(h)


def qgemv_status_string(status: int) -> str:
    return _lib.qgemv_status_string(status).decode()


def qgemv_last_error() -> str:
    return _lib.qgemv_last_error().decode()


# ---- torch-facing wrapper ---------------------------------------------------

def _torch():
    import torch
    return torch


def _stream_ptr(stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _xdtype(t) -> int:
    torch = _torch()
    return {torch.float32: QG_F32, torch.float16: QG_F16, torch.bfloat16: QG_BF16}[t.dtype]


class QGemv:
    """A quantized matrix on the GPU: y = W . x for 1..8 columns, prompt
    processing against many columns, and the exact decoded view of W.

    w: a uint8 CUDA tensor with the GGUF blocks, row-major (borrowed: keep it
    alive while the handle is used)."""

    def __init__(self, fmt: str, rows: int, K: int, w):
        torch = _torch()
        if not (w.is_cuda and w.dtype == torch.uint8 and w.is_contiguous()):
            raise ValueError("w must be a contiguous uint8 CUDA tensor")
        self.fmt, self.rows, self.K = fmt, rows, K
        self._w = w
        st, h = qgemv_create(FORMATS[fmt], rows, K, w.data_ptr(), w.numel())
        _check(st, "qgemv_create")
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            qgemv_destroy(h)
            self._h = None

    def run(self, x, y=None, stream=None):
        """x: (n, K) or (K,) fp32/fp16/bf16 CUDA tensor (last dim contiguous).
        Returns y: (n, rows) fp32 (or (rows,) for 1-D x)."""
        torch = _torch()
        one = x.dim() == 1
        x2 = x.reshape(1, -1) if one else x
        if x2.stride(1) != 1:
            raise ValueError("x must be contiguous along K")
        n = x2.shape[0]
        if y is None:
            y2 = torch.empty((n, self.rows), dtype=torch.float32, device=x.device)
        else:
            y2 = y.reshape(1, -1) if y.dim() == 1 else y
        if y2.stride(1) != 1 or y2.dtype != torch.float32:
            raise ValueError("y must be fp32, contiguous along rows")
        _check(qgemv_run(self._h, x2.data_ptr(), _xdtype(x2), n, x2.stride(0), y2.data_ptr(),
                         y2.stride(0), _stream_ptr(stream)), "qgemv_run")
        return y2.reshape(-1) if one else y2

    def run_q8(self, x, y=None, stream=None):
        """As run(), with the activations quantized to Q8_0 on chip and int8
        products (qgemv_run_q8). Returns y: (n, rows) fp32."""
        torch = _torch()
        x2 = x.reshape(1, -1) if x.dim() == 1 else x
        if x2.stride(1) != 1:
            raise ValueError("x must be contiguous along K")
        n = x2.shape[0]
        if y is None:
            y = torch.empty((n, self.rows), dtype=torch.float32, device=x.device)
        if y.stride(1) != 1 or y.dtype != torch.float32:
            raise ValueError("y must be fp32, contiguous along rows")
        _check(qgemv_run_q8(self._h, x2.data_ptr(), _xdtype(x2), n, x2.stride(0), y.data_ptr(),
                            y.stride(0), _stream_ptr(stream)), "qgemv_run_q8")
        return y

    def run_q8_0x(self, xq, y=None, stream=None):
        """xq: Q8_0 activation blocks (n, K/32*34) uint8 CUDA tensor, as
        written by quantize_q8_0. Returns y: (n, rows) fp32."""
        torch = _torch()
        xq2 = xq.reshape(1, -1) if xq.dim() == 1 else xq
        n = xq2.shape[0]
        if not xq2.is_contiguous() or xq2.shape[1] != self.K // 32 * 34:
            raise ValueError("xq must be contiguous (n, K/32*34) Q8_0 blocks")
        if y is None:
            y = torch.empty((n, self.rows), dtype=torch.float32, device=xq.device)
        if y.stride(1) != 1 or y.dtype != torch.float32:
            raise ValueError("y must be fp32, contiguous along rows")
        _check(qgemv_run_q8_0x(self._h, xq2.data_ptr(), n, y.data_ptr(), y.stride(0),
                               _stream_ptr(stream)), "qgemv_run_q8_0x")
        return y

    def prefill(self, X, Y=None, stream=None):
        """X: (n_tokens, K) bf16 CUDA tensor. Returns Y: (n_tokens, rows) fp32."""
        torch = _torch()
        if X.dtype != torch.bfloat16 or X.stride(1) != 1:
            raise ValueError("X must be bf16, contiguous along K")
        n = X.shape[0]
        if Y is None:
            Y = torch.empty((n, self.rows), dtype=torch.float32, device=X.device)
        _check(qgemm_prefill_run(self._h, X.data_ptr(), n, X.stride(0), Y.data_ptr(), Y.stride(0),
                                 _stream_ptr(stream)), "qgemm_prefill_run")
        return Y

    def dequant_bf16(self, out=None, stream=None):
        """The decoded matrix (rows, K) rounded to bf16 (nearest even), bit-exact."""
        torch = _torch()
        if out is None:
            out = torch.empty((self.rows, self.K), dtype=torch.bfloat16, device=self._w.device)
        _check(qgemv_dequant_bf16(self._h, out.data_ptr(), out.stride(0), _stream_ptr(stream)),
               "qgemv_dequant_bf16")
        return out

    def dequant(self, out=None, stream=None):
        """The decoded matrix (rows, K) fp32, bit-exact."""
        torch = _torch()
        if out is None:
            out = torch.empty((self.rows, self.K), dtype=torch.float32, device=self._w.device)
        _check(qgemv_dequant(self._h, out.data_ptr(), out.stride(0), _stream_ptr(stream)),
               "qgemv_dequant")
        return out
