"""ctypes view of the CPU oracle (oracle/qblk_oracle.c).

TEST INFRASTRUCTURE ONLY.  The oracle is a plain, single-threaded C
implementation of the block formats and their products, written from the
pages' definitions.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import it; the GPU library never does, and the two share
no code.  Arrays are numpy arrays in host memory.
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

Q4_0, SB4, SB4_AFFINE, Q4_K, W4G128 = 0, 1, 2, 3, 4
F32, F16, BF16 = 0, 1, 2

_lib = None


def lib():
    """Load (building first if it is missing) the oracle library."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = C.CDLL(_build.LIB)
        p, i64, i32 = C.c_void_p, C.c_int64, C.c_int
        L.orc_f16_to_f32.argtypes, L.orc_f16_to_f32.restype = [C.c_uint16], C.c_float
        L.orc_f32_to_f16.argtypes, L.orc_f32_to_f16.restype = [C.c_float], C.c_uint16
        L.orc_bf16_to_f32.argtypes, L.orc_bf16_to_f32.restype = [C.c_uint16], C.c_float
        L.orc_f32_to_bf16.argtypes, L.orc_f32_to_bf16.restype = [C.c_float], C.c_uint16
        L.orc_rha.argtypes, L.orc_rha.restype = [C.c_float], C.c_float
        L.orc_block_elems.argtypes, L.orc_block_elems.restype = [i32], i32
        L.orc_block_bytes.argtypes, L.orc_block_bytes.restype = [i32], i32
        L.orc_meta_int8.argtypes = [p, i32, C.c_float, p, p, p]
        L.orc_quantize_q4_0.argtypes = [p, i32, i64, i64, p]
        L.orc_quantize_q4_0_ref.argtypes = [p, i64, i64, p]
        L.orc_quantize_sb4.argtypes = [p, i32, i64, i64, i32, p]
        L.orc_quantize_q4_k.argtypes = [p, i32, i64, i64, p]
        L.orc_quantize_w4g128.argtypes = [p, i32, i64, i64, p]
        L.orc_quantize_act_i8.argtypes = [p, i32, i64, i64, p, p]
        L.orc_gemm_w4a8.argtypes = [p, i64, i64, p, p, i64, p, i64, p, p]
        L.orc_dequant.argtypes = [i32, p, i64, i64, p]
        L.orc_gemv.argtypes = [i32, p, i64, i64, p, p, i64, p, p]
        L.orc_gemm.argtypes = [i32, p, i64, i64, p, i64, p, i64, p, p]
        for f in ("orc_meta_int8", "orc_quantize_q4_0", "orc_quantize_q4_0_ref",
                  "orc_quantize_sb4", "orc_quantize_q4_k", "orc_quantize_w4g128",
                  "orc_quantize_act_i8", "orc_gemm_w4a8", "orc_dequant", "orc_gemv", "orc_gemm"):
            getattr(L, f).restype = i32
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(C.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def block_elems(fmt):
    return lib().orc_block_elems(fmt)


def block_bytes(fmt):
    return lib().orc_block_bytes(fmt)


def packed_bytes(fmt, rows, k):
    return rows * (k // block_elems(fmt)) * block_bytes(fmt)


def f16_to_f32(bits):
    return lib().orc_f16_to_f32(int(bits))


def f32_to_f16(v):
    return lib().orc_f32_to_f16(float(v))


def bf16_to_f32(bits):
    return lib().orc_bf16_to_f32(int(bits))


def f32_to_bf16(v):
    return lib().orc_f32_to_bf16(float(v))


def rha(v):
    return lib().orc_rha(float(v))


def meta_int8(scales, S_forced=0.0):
    """[K-quants blog, super-block steps 1-4] -> (codes int8[n], S16 bits, S used)."""
    s = np.ascontiguousarray(scales, dtype=np.float32)
    codes = np.zeros(s.size, dtype=np.int8)
    S16 = np.zeros(1, dtype=np.uint16)
    Su = np.zeros(1, dtype=np.float32)
    _check(lib().orc_meta_int8(_ptr(s), s.size, float(S_forced), _ptr(codes),
                               _ptr(S16), _ptr(Su)), "meta_int8")
    return codes, int(S16[0]), float(Su[0])


def _dense(w):
    """numpy array (f32, f16, or uint16 bf16 bits with dtype tag) -> (arr, tag)."""
    if isinstance(w, tuple):  # (uint16 array of bf16 bits, BF16)
        arr, tag = w
        return np.ascontiguousarray(arr, dtype=np.uint16), tag
    if w.dtype == np.float32:
        return np.ascontiguousarray(w), F32
    if w.dtype == np.float16:
        return np.ascontiguousarray(w), F16
    raise TypeError(f"unsupported dense dtype {w.dtype}")


def quantize_q4_0(w):
    arr, tag = _dense(w)
    rows, k = arr.shape
    out = np.zeros(packed_bytes(Q4_0, rows, k), dtype=np.uint8)
    _check(lib().orc_quantize_q4_0(_ptr(arr), tag, rows, k, _ptr(out)), "quantize_q4_0")
    return out


def quantize_q4_0_ref(w):
    arr = np.ascontiguousarray(w, dtype=np.float32)
    rows, k = arr.shape
    out = np.zeros(packed_bytes(Q4_0, rows, k), dtype=np.uint8)
    _check(lib().orc_quantize_q4_0_ref(_ptr(arr), rows, k, _ptr(out)), "quantize_q4_0_ref")
    return out


def quantize_sb4(w, affine=False):
    arr, tag = _dense(w)
    rows, k = arr.shape
    fmt = SB4_AFFINE if affine else SB4
    out = np.zeros(packed_bytes(fmt, rows, k), dtype=np.uint8)
    _check(lib().orc_quantize_sb4(_ptr(arr), tag, rows, k, int(bool(affine)), _ptr(out)),
           "quantize_sb4")
    return out


def quantize_q4_k(w):
    """Q4_0 chapter 4.6 form: fp16 d, dmin; 6-bit s_j, m_j; 4-bit codes."""
    arr, tag = _dense(w)
    rows, k = arr.shape
    out = np.zeros(packed_bytes(Q4_K, rows, k), dtype=np.uint8)
    _check(lib().orc_quantize_q4_k(_ptr(arr), tag, rows, k, _ptr(out)), "quantize_q4_k")
    return out


def quantize_w4g128(w):
    """TurboQuant article 2.1: per-row symmetric groups of 128, 4-bit (planar layout)."""
    arr, tag = _dense(w)
    rows, k = arr.shape
    out = np.zeros(packed_bytes(W4G128, rows, k), dtype=np.uint8)
    _check(lib().orc_quantize_w4g128(_ptr(arr), tag, rows, k, _ptr(out)), "quantize_w4g128")
    return out


def quantize_act_i8(x):
    """TurboQuant article 2.2: 8-bit activations, one symmetric scale per row (token).
    Returns (xq int8 n x k, scale float32 n)."""
    arr, tag = _dense(x)
    n, k = arr.shape
    xq = np.zeros((n, k), dtype=np.int8)
    sc = np.zeros(n, dtype=np.float32)
    _check(lib().orc_quantize_act_i8(_ptr(arr), tag, n, k, _ptr(xq), _ptr(sc)), "quantize_act_i8")
    return xq, sc


def gemm_w4a8(blocks, m, k, xq, scale, rows=None):
    """fp64 Y (n x nrows) of the rebuilt weights times the rebuilt activations, and the bound."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8)
    q = np.ascontiguousarray(xq, dtype=np.int8)
    s = np.ascontiguousarray(scale, dtype=np.float32)
    n = q.shape[0]
    assert q.shape[1] == k and s.size == n
    if rows is None:
        idx, nr = None, m
    else:
        idx = np.ascontiguousarray(rows, dtype=np.int64)
        nr = idx.size
    Y = np.zeros((n, nr), dtype=np.float64)
    B = np.zeros((n, nr), dtype=np.float64)
    _check(lib().orc_gemm_w4a8(_ptr(b), m, k, _ptr(q), _ptr(s), n,
                               _ptr(idx) if idx is not None else None, nr, _ptr(Y), _ptr(B)),
           "gemm_w4a8")
    return Y, B


def quantize(fmt, w):
    if fmt == Q4_0:
        return quantize_q4_0(w)
    if fmt == W4G128:
        return quantize_w4g128(w)
    if fmt == Q4_K:
        return quantize_q4_k(w)
    return quantize_sb4(w, affine=(fmt == SB4_AFFINE))


def dequant(fmt, blocks, rows, k):
    b = np.ascontiguousarray(blocks, dtype=np.uint8)
    if b.size < packed_bytes(fmt, rows, k):
        raise ValueError("block buffer too small")
    out = np.zeros((rows, k), dtype=np.float32)
    _check(lib().orc_dequant(fmt, _ptr(b), rows, k, _ptr(out)), "dequant")
    return out


def gemv(fmt, blocks, m, k, x, rows=None):
    """fp64 y and bound sum|w x| for the listed rows (all rows if None)."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8)
    xd = np.ascontiguousarray(x, dtype=np.float64)
    assert xd.size == k
    if rows is None:
        idx, n = None, m
    else:
        idx = np.ascontiguousarray(rows, dtype=np.int64)
        n = idx.size
    y = np.zeros(n, dtype=np.float64)
    bound = np.zeros(n, dtype=np.float64)
    _check(lib().orc_gemv(fmt, _ptr(b), m, k, _ptr(xd),
                          _ptr(idx) if idx is not None else None, n, _ptr(y), _ptr(bound)),
           "gemv")
    return y, bound


def gemm(fmt, blocks, m, k, X, rows=None):
    """X: n x k; returns fp64 Y (n x nrows) and the bound of the same shape."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8)
    Xd = np.ascontiguousarray(X, dtype=np.float64)
    n = Xd.shape[0]
    assert Xd.shape[1] == k
    if rows is None:
        idx, nr = None, m
    else:
        idx = np.ascontiguousarray(rows, dtype=np.int64)
        nr = idx.size
    Y = np.zeros((n, nr), dtype=np.float64)
    B = np.zeros((n, nr), dtype=np.float64)
    _check(lib().orc_gemm(fmt, _ptr(b), m, k, _ptr(Xd), n,
                          _ptr(idx) if idx is not None else None, nr, _ptr(Y), _ptr(B)),
           "gemm")
    return Y, B
