"""Python binding of libqblk (the gfx950 C-ABI library), via ctypes.

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch supplies device memory and the stream; tensors must live on a GPU.
If the library is not built this module raises on import -- there is no CPU
fallback.  Build with ``python bit_block_quant_amd/build.py`` (or ``__graft_entry__.build()``).

    blocks = qblk.quantize(w, qblk.SB4)          # w: (rows, k) f32/f16/bf16
    y      = qblk.gemv(blocks, qblk.SB4, m, k, x) # x: (k,) f32/f16/bf16 -> (m,) f32
    Y      = qblk.gemm(blocks, qblk.SB4, m, k, X) # X: (n, k) bf16 -> (n, m) f32
    W      = qblk.dequant(blocks, qblk.SB4, m, k, torch.float32)
    xq, s  = qblk.quantize_act_i8(X)             # W4A8: int8 tokens + fp32 scales
    Y      = qblk.gemm_w4a8(qblk.quantize(w, qblk.W4G128), m, k, xq, s)
"""
import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqblk.so")

Q4_0, SB4, SB4_AFFINE, Q4_K, W4G128 = 0, 1, 2, 3, 4
F32, F16, BF16 = 0, 1, 2
FORMATS = {"q4_0": Q4_0, "sb4": SB4, "sb4_affine": SB4_AFFINE, "q4_k": Q4_K, "w4g128": W4G128}
_DT = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}

STATUS = {
    0: "QBLK_OK", 1: "QBLK_ERR_NULL", 2: "QBLK_ERR_SHAPE", 3: "QBLK_ERR_DTYPE",
    4: "QBLK_ERR_ALIGN", 5: "QBLK_ERR_UNSUPPORTED", 6: "QBLK_ERR_LAUNCH", 7: "QBLK_ERR_FORMAT",
}

# every symbol include/qblk.h declares
EXPORTS = (
    "qblk_block_bytes", "qblk_block_elems", "qblk_packed_bytes", "qblk_quantize_q4_0",
    "qblk_quantize_q4_0_ref", "qblk_quantize_sb4", "qblk_quantize_q4_k", "qblk_quantize_w4g128",
    "qblk_quantize_act_i8", "qblk_dequant", "qblk_gemv", "qblk_gemm", "qblk_gemm_w4a8",
    "qblk_status_string", "qblk_version",
)


class QblkError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({_lib.qblk_status_string(status).decode()})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libqblk.so not found at {LIB_PATH}; build it with `python bit_block_quant_amd/build.py`")
    L = C.CDLL(LIB_PATH)
    p, i64, i32 = C.c_void_p, C.c_int64, C.c_int
    L.qblk_block_bytes.argtypes, L.qblk_block_bytes.restype = [i32], C.c_size_t
    L.qblk_block_elems.argtypes, L.qblk_block_elems.restype = [i32], i32
    L.qblk_packed_bytes.argtypes, L.qblk_packed_bytes.restype = [i32, i64, i64], C.c_size_t
    L.qblk_quantize_q4_0.argtypes = [p, i32, i64, i64, p, p]
    L.qblk_quantize_q4_0_ref.argtypes = [p, i32, i64, i64, p, p]
    L.qblk_quantize_sb4.argtypes = [p, i32, i64, i64, i32, p, p]
    L.qblk_quantize_q4_k.argtypes = [p, i32, i64, i64, p, p]
    L.qblk_quantize_w4g128.argtypes = [p, i32, i64, i64, p, p]
    L.qblk_quantize_act_i8.argtypes = [p, i32, i64, i64, p, p, p]
    L.qblk_gemm_w4a8.argtypes = [p, i64, i64, p, p, i64, p, p]
    L.qblk_dequant.argtypes = [i32, p, i64, i64, p, i32, p]
    L.qblk_gemv.argtypes = [i32, p, i64, i64, p, i32, p, p]
    L.qblk_gemm.argtypes = [i32, p, i64, i64, p, i32, i64, p, p]
    for f in ("qblk_quantize_q4_0", "qblk_quantize_q4_0_ref", "qblk_quantize_sb4", "qblk_quantize_q4_k",
              "qblk_quantize_w4g128", "qblk_quantize_act_i8", "qblk_dequant", "qblk_gemv", "qblk_gemm",
              "qblk_gemm_w4a8"):
        getattr(L, f).restype = i32
    L.qblk_status_string.argtypes, L.qblk_status_string.restype = [i32], C.c_char_p
    L.qblk_version.argtypes, L.qblk_version.restype = [], C.c_char_p
    return L


_lib = _load()


def lib():
    return _lib


def version():
    return _lib.qblk_version().decode()


def block_bytes(fmt):
    return _lib.qblk_block_bytes(fmt)


def block_elems(fmt):
    return _lib.qblk_block_elems(fmt)


def packed_bytes(fmt, rows, k):
    return _lib.qblk_packed_bytes(fmt, rows, k)


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else C.c_void_p(0)


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _check(st, what):
    if st != 0:
        raise QblkError(st, what)


def _dtype(t):
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported element type {t.dtype}") from None


def quantize(w, fmt, out=None, stream=None, ref=False):
    """Quantize a (rows, k) device tensor into a uint8 tensor of packed blocks.

    ref=True (Q4_0 only) uses the Q4_0 chapter's signed max/-8 quantizer."""
    rows, k = w.shape
    nbytes = packed_bytes(fmt, rows, k)
    if out is None:
        out = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=w.device)
    if fmt == Q4_0:
        f = _lib.qblk_quantize_q4_0_ref if ref else _lib.qblk_quantize_q4_0
        _check(f(_ptr(w), _dtype(w), rows, k, _ptr(out), _stream(stream)), "qblk_quantize_q4_0")
    elif fmt == Q4_K:
        _check(_lib.qblk_quantize_q4_k(_ptr(w), _dtype(w), rows, k, _ptr(out), _stream(stream)),
               "qblk_quantize_q4_k")
    elif fmt == W4G128:
        _check(_lib.qblk_quantize_w4g128(_ptr(w), _dtype(w), rows, k, _ptr(out), _stream(stream)),
               "qblk_quantize_w4g128")
    else:
        _check(_lib.qblk_quantize_sb4(_ptr(w), _dtype(w), rows, k, int(fmt == SB4_AFFINE), _ptr(out),
                                      _stream(stream)), "qblk_quantize_sb4")
    return out[:nbytes] if nbytes else out[:0]


def dequant(blocks, fmt, rows, k, dtype=torch.float32, out=None, stream=None):
    if out is None:
        out = torch.empty((rows, k), dtype=dtype, device=blocks.device)
    _check(_lib.qblk_dequant(fmt, _ptr(blocks), rows, k, _ptr(out), _dtype(out), _stream(stream)),
           "qblk_dequant")
    return out


def gemv(blocks, fmt, m, k, x, out=None, stream=None):
    if out is None:
        out = torch.empty(m, dtype=torch.float32, device=x.device)
    _check(_lib.qblk_gemv(fmt, _ptr(blocks), m, k, _ptr(x), _dtype(x), _ptr(out), _stream(stream)),
           "qblk_gemv")
    return out


def gemm(blocks, fmt, m, k, X, out=None, stream=None):
    n = X.shape[0]
    if out is None:
        out = torch.empty((n, m), dtype=torch.float32, device=X.device)
    _check(_lib.qblk_gemm(fmt, _ptr(blocks), m, k, _ptr(X), _dtype(X), n, _ptr(out),
                          _stream(stream)), "qblk_gemm")
    return out


def quantize_act_i8(x, out=None, scale=None, stream=None):
    """8-bit activations: (n, k) f32/f16/bf16 -> (int8 codes (n, k), fp32 scales (n,))."""
    n, k = x.shape
    if out is None:
        out = torch.empty((n, k), dtype=torch.int8, device=x.device)
    if scale is None:
        scale = torch.empty(n, dtype=torch.float32, device=x.device)
    _check(_lib.qblk_quantize_act_i8(_ptr(x), _dtype(x), n, k, _ptr(out), _ptr(scale), _stream(stream)),
           "qblk_quantize_act_i8")
    return out, scale


def gemm_w4a8(blocks, m, k, xq, scale, out=None, stream=None):
    """Y (n, m) fp32 = the W4A8 product of QBLK_W4G128 blocks and int8 activations."""
    n = xq.shape[0]
    if out is None:
        out = torch.empty((n, m), dtype=torch.float32, device=xq.device)
    _check(_lib.qblk_gemm_w4a8(_ptr(blocks), m, k, _ptr(xq), _ptr(scale), n, _ptr(out), _stream(stream)),
           "qblk_gemm_w4a8")
    return out
