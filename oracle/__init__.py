"""ConvRot W8A8 reference oracle -- TEST INFRASTRUCTURE ONLY.

A numpy-facing wrapper over ``liboracle.so`` (plain C, built by ``oracle/build.py``
with gcc).  Only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import this package.  The product library never loads it and shares no
code with it.

Every function follows the method as the pages state it (see ``oracle.c`` for the
citations and the readings taken where the pages are silent).  Arrays are numpy,
row-major, contiguous; bf16 values travel as ``uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

BLOCK = 128


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = C.CDLL(_LIB_PATH)
        p = C.c_void_p
        i64 = C.c_int64
        i32 = C.c_int
        L.oracle_hadamard.argtypes = [i32, p]
        L.oracle_norm_const.argtypes = [i32]
        L.oracle_norm_const.restype = C.c_double
        L.oracle_rotate_rows.argtypes = [p, i64, i64, i32, p, p]
        L.oracle_quantize_rows.argtypes = [p, i64, i64, p, p]
        L.oracle_rotate_quantize.argtypes = [p, i64, i64, i32, i64, p, p, p]
        L.oracle_gemm_i8_i32.argtypes = [p, p, i64, i64, i64, p, i64, p]
        L.oracle_dequant_epilogue.argtypes = [p, i64, i64, p, p, p, p, p]
        L.oracle_bwd_quant_dy.argtypes = [p, i64, i64, p, p, p]
        L.oracle_gemm_i8_i32_rows_of_b.argtypes = [p, p, i64, i64, i64, p, i64, p]
        L.oracle_bwd_int8_epilogue.argtypes = [p, i64, i64, p, p, i32, p]
        L.oracle_dequant_weight.argtypes = [p, p, i64, i64, i32, p]
        L.oracle_bf16_gemm_dx.argtypes = [p, p, i64, i64, i64, p, i64, p]
        L.oracle_embedding_lookup.argtypes = [p, i64, p, p, i64, i64, i32, p, p]
        L.oracle_lora_down.argtypes = [p, i64, i64, p, i64, p, i64, p]
        L.oracle_lora_epilogue.argtypes = [p, i64, i64, p, p, p, p, p, p, i64, C.c_double, p]
        L.oracle_double_to_bf16.argtypes = [C.c_double]
        L.oracle_double_to_bf16.restype = C.c_uint16
        L.oracle_rne_integer.argtypes = [C.c_double]
        L.oracle_rne_integer.restype = C.c_double
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = C.c_int
        L.oracle_set_num_threads.argtypes = [C.c_int]
        L.oracle_set_num_threads.restype = None
        for name in ("oracle_hadamard", "oracle_rotate_rows", "oracle_quantize_rows",
                     "oracle_rotate_quantize", "oracle_gemm_i8_i32", "oracle_dequant_epilogue",
                     "oracle_bwd_quant_dy", "oracle_gemm_i8_i32_rows_of_b",
                     "oracle_bwd_int8_epilogue", "oracle_dequant_weight", "oracle_bf16_gemm_dx",
                     "oracle_embedding_lookup"):
            getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _rows_arg(rows, M):
    if rows is None:
        return None, M
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if r.size and (r.min() < 0 or r.max() >= M):
        raise IndexError("row index out of range")
    return r, int(r.size)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what}: oracle rejected the arguments (rc={rc})")


# --------------------------------------------------------------------------
# O1
# --------------------------------------------------------------------------

def hadamard(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix H_n (entries +-1, natural order), int8."""
    H = np.empty((n, n), dtype=np.int8)
    _check(lib().oracle_hadamard(n, _ptr(H)), "hadamard")
    return H


def norm_const(block: int = BLOCK) -> float:
    """The binary64 constant 1/sqrt(block) used by the normalised rotation."""
    return lib().oracle_norm_const(block)


# --------------------------------------------------------------------------
# O2 - O6
# --------------------------------------------------------------------------

def rotate_rows(x_bf16: np.ndarray, block: int = BLOCK):
    """Rotated rows r = fl32(fl64(S * c)); returns (r float32, inexact_row_count)."""
    x = _c(x_bf16, np.uint16)
    rows, cols = x.shape
    r = np.empty((rows, cols), dtype=np.float32)
    bad = C.c_int64(0)
    _check(lib().oracle_rotate_rows(_ptr(x), rows, cols, block, _ptr(r), C.byref(bad)),
           "rotate_rows")
    return r, int(bad.value)


def quantize_rows(r: np.ndarray):
    """Symmetric per-row int8 of fp32 rows: (codes int8, scales float32)."""
    r = _c(r, np.float32)
    rows, cols = r.shape
    q = np.empty((rows, cols), dtype=np.int8)
    s = np.empty((rows,), dtype=np.float32)
    _check(lib().oracle_quantize_rows(_ptr(r), rows, cols, _ptr(q), _ptr(s)), "quantize_rows")
    return q, s


def rotate_quantize(x_bf16: np.ndarray, block: int = BLOCK, chunk_rows: int = 0):
    """Rotate then quantize every row (weights at load, activations online, the
    embedding in row chunks).  Returns (codes, scales, inexact_row_count)."""
    x = _c(x_bf16, np.uint16)
    rows, cols = x.shape
    q = np.empty((rows, cols), dtype=np.int8)
    s = np.empty((rows,), dtype=np.float32)
    bad = C.c_int64(0)
    _check(lib().oracle_rotate_quantize(_ptr(x), rows, cols, block, chunk_rows, _ptr(q), _ptr(s),
                                        C.byref(bad)), "rotate_quantize")
    return q, s, int(bad.value)


# --------------------------------------------------------------------------
# O7, O8
# --------------------------------------------------------------------------

def gemm_i8_i32(a: np.ndarray, b: np.ndarray, rows=None) -> np.ndarray:
    """acc[i, n] = sum_k a[rows[i], k] * b[n, k] (int32)."""
    a = _c(a, np.int8)
    b = _c(b, np.int8)
    M, K = a.shape
    N, K2 = b.shape
    assert K == K2
    r, nr = _rows_arg(rows, M)
    acc = np.empty((nr, N), dtype=np.int32)
    _check(lib().oracle_gemm_i8_i32(_ptr(a), _ptr(b), M, N, K, _ptr(r), nr, _ptr(acc)), "gemm")
    return acc


def dequant_epilogue(acc, sx, sw, rows=None, bias=None) -> np.ndarray:
    acc = _c(acc, np.int32)
    sx = _c(sx, np.float32)
    sw = _c(sw, np.float32)
    nr, N = acc.shape
    r = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if bias is not None:
        bias = _c(bias, np.uint16)
    y = np.empty((nr, N), dtype=np.uint16)
    _check(lib().oracle_dequant_epilogue(_ptr(acc), nr, N, _ptr(sx), _ptr(r), _ptr(sw),
                                         _ptr(bias), _ptr(y)), "dequant_epilogue")
    return y


def linear_fwd(x_bf16, qw, sw, bias=None, rows=None, block: int = BLOCK):
    """Forward of the ConvRot linear: rotate + quantize x per row, int8 GEMM
    with q_w, dequantize.  Returns dict(qx, sx, acc, y) (acc, y for ``rows``)."""
    qx, sx, bad = rotate_quantize(x_bf16, block)
    acc = gemm_i8_i32(qx, qw, rows)
    y = dequant_epilogue(acc, sx, sw, rows, bias)
    return dict(qx=qx, sx=sx, acc=acc, y=y, inexact_rows=bad)


# --------------------------------------------------------------------------
# O13: LoRA branch of the forward
# --------------------------------------------------------------------------

def lora_down(x_bf16, a_bf16, rows=None) -> np.ndarray:
    """xa = bf16(x . A^T) (binary64 sum) for the listed rows of x; A is [R, K]."""
    x = _c(x_bf16, np.uint16)
    a = _c(a_bf16, np.uint16)
    M, K = x.shape
    R, Ka = a.shape
    assert Ka == K
    r = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    nr = M if r is None else r.size
    xa = np.empty((nr, R), dtype=np.uint16)
    _check(lib().oracle_lora_down(_ptr(x), M, K, _ptr(a), R, _ptr(r), nr, _ptr(xa)), "lora_down")
    return xa


def lora_epilogue(acc, sx, sw, xa, b_bf16, scale: float, rows=None, bias=None) -> np.ndarray:
    """y = bf16(acc*s_x*s_w + bias + scale * xa . B^T), binary64, one rounding."""
    acc = _c(acc, np.int32)
    sx = _c(sx, np.float32)
    sw = _c(sw, np.float32)
    xa = _c(xa, np.uint16)
    b = _c(b_bf16, np.uint16)
    nr, N = acc.shape
    R = xa.shape[1]
    assert b.shape == (N, R) and xa.shape[0] == nr
    r = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if bias is not None:
        bias = _c(bias, np.uint16)
    y = np.empty((nr, N), dtype=np.uint16)
    _check(lib().oracle_lora_epilogue(_ptr(acc), nr, N, _ptr(sx), _ptr(r), _ptr(sw), _ptr(bias),
                                      _ptr(xa), _ptr(b), R, C.c_double(scale), _ptr(y)),
           "lora_epilogue")
    return y


# --------------------------------------------------------------------------
# O9, O10
# --------------------------------------------------------------------------

def bwd_quant_dy(dy_bf16, sw):
    dy = _c(dy_bf16, np.uint16)
    sw = _c(sw, np.float32)
    M, N = dy.shape
    qg = np.empty((M, N), dtype=np.int8)
    sg = np.empty((M,), dtype=np.float32)
    _check(lib().oracle_bwd_quant_dy(_ptr(dy), M, N, _ptr(sw), _ptr(qg), _ptr(sg)),
           "bwd_quant_dy")
    return qg, sg


def gemm_i8_i32_rows_of_b(qg, qw, rows=None):
    """acc2[i, k] = sum_n qg[rows[i], n] * qw[n, k]."""
    qg = _c(qg, np.int8)
    qw = _c(qw, np.int8)
    M, N = qg.shape
    N2, K = qw.shape
    assert N == N2
    r, nr = _rows_arg(rows, M)
    acc2 = np.empty((nr, K), dtype=np.int32)
    _check(lib().oracle_gemm_i8_i32_rows_of_b(_ptr(qg), _ptr(qw), M, N, K, _ptr(r), nr,
                                              _ptr(acc2)), "gemm_rows_of_b")
    return acc2


def bwd_int8_epilogue(acc2, sg, rows=None, block: int = BLOCK):
    acc2 = _c(acc2, np.int32)
    sg = _c(sg, np.float32)
    nr, K = acc2.shape
    r = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    dx = np.empty((nr, K), dtype=np.uint16)
    _check(lib().oracle_bwd_int8_epilogue(_ptr(acc2), nr, K, _ptr(sg), _ptr(r), block, _ptr(dx)),
           "bwd_int8_epilogue")
    return dx


def bwd_dx_int8(dy_bf16, qw, sw, rows=None, block: int = BLOCK):
    qg, sg = bwd_quant_dy(dy_bf16, sw)
    acc2 = gemm_i8_i32_rows_of_b(qg, qw, rows)
    dx = bwd_int8_epilogue(acc2, sg, rows, block)
    return dict(qg=qg, sg=sg, acc2=acc2, dx=dx)


def dequant_weight(qw, sw, block: int = BLOCK):
    qw = _c(qw, np.int8)
    sw = _c(sw, np.float32)
    N, K = qw.shape
    what = np.empty((N, K), dtype=np.uint16)
    _check(lib().oracle_dequant_weight(_ptr(qw), _ptr(sw), N, K, block, _ptr(what)),
           "dequant_weight")
    return what


def bf16_gemm_dx(dy_bf16, what, rows=None):
    dy = _c(dy_bf16, np.uint16)
    what = _c(what, np.uint16)
    M, N = dy.shape
    N2, K = what.shape
    assert N == N2
    r, nr = _rows_arg(rows, M)
    dx = np.empty((nr, K), dtype=np.uint16)
    _check(lib().oracle_bf16_gemm_dx(_ptr(dy), _ptr(what), M, N, K, _ptr(r), nr, _ptr(dx)),
           "bf16_gemm_dx")
    return dx


def bwd_dx_bf16(dy_bf16, qw, sw, rows=None, block: int = BLOCK):
    what = dequant_weight(qw, sw, block)
    return dict(what=what, dx=bf16_gemm_dx(dy_bf16, what, rows))


# --------------------------------------------------------------------------
# O11
# --------------------------------------------------------------------------

def embedding_lookup(ids, qe, se, block: int = BLOCK):
    ids = _c(ids, np.int32)
    qe = _c(qe, np.int8)
    se = _c(se, np.float32)
    V, D = qe.shape
    T = ids.shape[0]
    out = np.empty((T, D), dtype=np.uint16)
    oob = C.c_int64(0)
    _check(lib().oracle_embedding_lookup(_ptr(ids), T, _ptr(qe), _ptr(se), V, D, block, _ptr(out),
                                         C.byref(oob)), "embedding_lookup")
    return out, int(oob.value)


# --------------------------------------------------------------------------
# Rounding helpers (pinned by the oracle's own tests)
# --------------------------------------------------------------------------

def num_threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for the following oracle calls (timings only; results do not
    depend on the thread count)."""
    lib().oracle_set_num_threads(int(n))


def double_to_bf16(x: float) -> int:
    return int(lib().oracle_double_to_bf16(float(x)))


def rne_integer(t: float) -> float:
    return float(lib().oracle_rne_integer(float(t)))
