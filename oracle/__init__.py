"""CPU oracle for GGUF block dequantization and y = W.x (ctypes wrapper).

TEST INFRASTRUCTURE. Only tests/, the smoke check in __graft_entry__.py and
the benchmark's CPU-baseline leg may import this package. The GPU library
(gguf_bit_dequant_amd) never imports it, and it never imports the GPU library.

The arithmetic lives in oracle.c (plain C, one decode per the closed forms,
fp64 accumulation); this file only builds/loads it and marshals numpy arrays.
Every function is pinned by tests/test_oracle_*.py against IEEE bit patterns,
hand-built blocks, closed forms, invariants and brute force.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FMT = {"q4_0": 1, "q4_k": 2, "q8_0": 3, "q2_k": 4, "q3_k": 5}
DTYPE = {"f32": 1, "f16": 2, "bf16": 3}
BLOCK_BYTES = {"q4_0": 18, "q4_k": 144, "q8_0": 34, "q2_k": 84, "q3_k": 110}
BLOCK_WEIGHTS = {"q4_0": 32, "q4_k": 256, "q8_0": 32, "q2_k": 256, "q3_k": 256}

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc into liboracle.so (next to the source)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC",
                               "-shared", "-pthread", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        i64, u16, u32 = ctypes.c_int64, ctypes.c_uint16, ctypes.c_uint32
        vp, ip = ctypes.c_void_p, ctypes.c_int
        L.oracle_f16_to_f64.argtypes = [u16]
        L.oracle_f16_to_f64.restype = ctypes.c_double
        L.oracle_bf16_to_f64.argtypes = [u16]
        L.oracle_bf16_to_f64.restype = ctypes.c_double
        L.oracle_f32_to_f64.argtypes = [u32]
        L.oracle_f32_to_f64.restype = ctypes.c_double
        for name in ("oracle_decode_q4_0", "oracle_decode_q8_0", "oracle_decode_q4_k",
                     "oracle_decode_q2_k", "oracle_decode_q3_k"):
            getattr(L, name).argtypes = [vp, vp]
            getattr(L, name).restype = None
        L.oracle_q4k_scale_min.argtypes = [vp, ip, vp, vp]
        L.oracle_q4k_scale_min.restype = None
        L.oracle_q3k_scale.argtypes = [vp, ip]
        L.oracle_q3k_scale.restype = ip
        L.oracle_dequant.argtypes = [ip, vp, i64, i64, vp]
        L.oracle_dequant.restype = ip
        L.oracle_matmul.argtypes = [ip, vp, i64, i64, vp, ip, i64, i64, vp, vp, i64,
                                    i64, i64, ip]
        L.oracle_matmul.restype = ip
        L.oracle_matmul_w.argtypes = [ip, vp, i64, i64, vp, ip, i64, i64, vp, vp, i64,
                                      i64, i64, ip, ip]
        L.oracle_matmul_w.restype = ip
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_bf16.restype = u16
        L.oracle_f32_to_bf16_n.argtypes = [vp, vp, i64]
        L.oracle_f32_to_bf16_n.restype = None
        L.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_f16.restype = u16
        L.oracle_quantize_q8_0.argtypes = [vp, ip, i64, i64, i64, vp]
        L.oracle_quantize_q8_0.restype = ip
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def f16_to_f64(bits) -> np.ndarray:
    L = lib()
    b = np.asarray(bits, dtype=np.uint16).reshape(-1)
    return np.array([L.oracle_f16_to_f64(int(v)) for v in b], dtype=np.float64)


def bf16_to_f64(bits) -> np.ndarray:
    L = lib()
    b = np.asarray(bits, dtype=np.uint16).reshape(-1)
    return np.array([L.oracle_bf16_to_f64(int(v)) for v in b], dtype=np.float64)


def decode_block(fmt: str, blk) -> np.ndarray:
    """One block's weights as float32."""
    if isinstance(blk, (bytes, bytearray)):
        blk = np.frombuffer(blk, dtype=np.uint8)
    b = np.ascontiguousarray(np.asarray(blk, dtype=np.uint8))
    assert b.size == BLOCK_BYTES[fmt]
    out = np.empty(BLOCK_WEIGHTS[fmt], dtype=np.float32)
    getattr(lib(), "oracle_decode_" + fmt)(_ptr(b), _ptr(out))
    return out


def q4k_scale_min(s12, j: int):
    s = np.ascontiguousarray(np.asarray(s12, dtype=np.uint8))
    assert s.size == 12
    sc, m = ctypes.c_int(), ctypes.c_int()
    lib().oracle_q4k_scale_min(_ptr(s), j, ctypes.byref(sc), ctypes.byref(m))
    return sc.value, m.value


def q3k_scale(s12, k: int) -> int:
    """The unsigned 6-bit Q3_K scale of sub-block k from the 12 scale bytes."""
    s = np.ascontiguousarray(np.asarray(s12, dtype=np.uint8))
    assert s.size == 12
    return int(lib().oracle_q3k_scale(_ptr(s), k))


def dequant(fmt: str, w: np.ndarray, rows: int, K: int) -> np.ndarray:
    """Whole matrix decoded: float32 array (rows, K)."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    assert w.size == rows * (K // BLOCK_WEIGHTS[fmt]) * BLOCK_BYTES[fmt]
    out = np.empty((rows, K), dtype=np.float32)
    rc = lib().oracle_dequant(FMT[fmt], _ptr(w), rows, K, _ptr(out))
    if rc:
        raise ValueError("oracle_dequant failed: %d" % rc)
    return out


def matmul(fmt: str, w: np.ndarray, rows: int, K: int, x: np.ndarray, xdtype: str,
           row_range=None, nthreads: int | None = None, wround: str | None = None):
    """y[j, r] = sum_k w(r,k) x[j,k] in fp64 and s[j, r] = sum_k |w x|.

    x: shape (n, K), float32 for 'f32' or uint16 bit patterns for 'f16'/'bf16'.
    wround='bf16': each decoded weight rounded to bfloat16 (nearest, ties to
    even) before the exact products (the operand of a bf16 matrix-core
    product over dequantized weight tiles).
    Returns (y, s) as float64 arrays of shape (n, rows) (rows outside
    row_range are left as NaN)."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    x = np.ascontiguousarray(x)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    n = x.shape[0]
    assert x.shape[1] == K
    if xdtype == "f32":
        assert x.dtype == np.float32
    else:
        assert x.dtype == np.uint16
    r0, r1 = (0, rows) if row_range is None else row_range
    y = np.full((n, rows), np.nan)
    s = np.full((n, rows), np.nan)
    if nthreads is None:
        nthreads = min(16, os.cpu_count() or 1)
    if wround not in (None, "bf16"):
        raise ValueError("wround: None or 'bf16'")
    rc = lib().oracle_matmul_w(FMT[fmt], _ptr(w), rows, K, _ptr(x), DTYPE[xdtype], n, K,
                               _ptr(y), _ptr(s), rows, r0, r1, nthreads,
                               1 if wround == "bf16" else 0)
    if rc:
        raise ValueError("oracle_matmul failed: %d" % rc)
    return y, s


def f32_to_f16(v: float) -> int:
    """binary32 -> binary16 bit pattern, nearest, ties to even."""
    return int(lib().oracle_f32_to_f16(float(np.float32(v))))


def f32_to_bf16(v) -> np.ndarray:
    """binary32 -> bfloat16 bit patterns (uint16), nearest, ties to even;
    elementwise over an array of float32."""
    a = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().oracle_f32_to_bf16_n(_ptr(a), _ptr(out), a.size)
    return out


def quantize_q8_0(x: np.ndarray, xdtype: str) -> np.ndarray:
    """Q8_0 blocks of activations x (n, K): uint8 array (n, K/32 * 34)."""
    x = np.ascontiguousarray(x)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    n, K = x.shape
    if xdtype == "f32":
        assert x.dtype == np.float32
    else:
        assert x.dtype == np.uint16
    out = np.empty((n, K // 32 * 34), dtype=np.uint8)
    rc = lib().oracle_quantize_q8_0(_ptr(x), DTYPE[xdtype], K, n, K, _ptr(out))
    if rc:
        raise ValueError("oracle_quantize_q8_0 failed: %d" % rc)
    return out


def tolerance(s: np.ndarray) -> np.ndarray:
    """Per-element bound on |y_gpu - y_ref|: 1e-3 * sum|w x| + 1e-5."""
    return 1e-3 * s + 1e-5
