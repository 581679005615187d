"""Python binding of libqblk (the gfx950 C-ABI library), via ctypes.

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch supplies device memory and the stream; tensors must live on the
current GPU and be contiguous, and every buffer must be large enough for the
call -- the C ABI cannot see extents, so these are checked here and a bad
argument raises ValueError/TypeError before anything is launched.
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
    "qblk_quantize_act_i8", "qblk_dequant", "qblk_gemv", "qblk_gemv_batch", "qblk_gemm", "qblk_gemm_w4a8",
    "qblk_set_deterministic", "qblk_deterministic", "qblk_status_string", "qblk_version",
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
    L.qblk_gemv_batch.argtypes = [i32, i64, i32, p, i32, p]
    L.qblk_gemm.argtypes = [i32, p, i64, i64, p, i32, i64, p, p]
    for f in ("qblk_quantize_q4_0", "qblk_quantize_q4_0_ref", "qblk_quantize_sb4", "qblk_quantize_q4_k",
              "qblk_quantize_w4g128", "qblk_quantize_act_i8", "qblk_dequant", "qblk_gemv", "qblk_gemm",
              "qblk_gemm_w4a8"):
        getattr(L, f).restype = i32
    L.qblk_status_string.argtypes, L.qblk_status_string.restype = [i32], C.c_char_p
    L.qblk_version.argtypes, L.qblk_version.restype = [], C.c_char_p
    L.qblk_set_deterministic.argtypes, L.qblk_set_deterministic.restype = [i32], i32
    L.qblk_deterministic.argtypes, L.qblk_deterministic.restype = [], i32
    return L


_lib = _load()


def lib():
    return _lib


def version():
    return _lib.qblk_version().decode()


def set_deterministic(on=True):
    """Reproducible products (qblk_set_deterministic): gemm and gemm_w4a8 stop
    splitting K over workgroups, so equal inputs give bitwise equal outputs."""
    _check(_lib.qblk_set_deterministic(1 if on else 0), "qblk_set_deterministic")


def deterministic():
    return bool(_lib.qblk_deterministic())


def block_bytes(fmt):
    return _lib.qblk_block_bytes(fmt)


def block_elems(fmt):
    return _lib.qblk_block_elems(fmt)


def packed_bytes(fmt, rows, k):
    return _lib.qblk_packed_bytes(fmt, rows, k)


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else C.c_void_p(0)


# ---------------------------------------------------------------- checks
# The C ABI sees raw pointers only, so the extents of every buffer are checked
# here, before any call: a short or strided tensor would make a kernel read or
# write past its allocation.  Each check raises ValueError (or TypeError for
# an element type) and nothing is launched.
_FLOAT_IN = (torch.float32, torch.float16, torch.bfloat16)


def _need(t, name, dtypes=None, min_numel=None, numel=None, ndim=None, dim1=None, device=None):
    """Validate one tensor argument; returns its device.  `device`: the device
    every other argument of the call lives on (None for the first one)."""
    if not isinstance(t, torch.Tensor) and not hasattr(t, "is_cuda"):
        raise TypeError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor (got device {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, the other arguments on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous (the kernels index it as a dense row-major array)")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name}: element type {t.dtype}, expected one of {[str(d) for d in dtypes]}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dimensions, got shape {tuple(t.shape)}")
    if dim1 is not None and t.shape[1] != dim1:
        raise ValueError(f"{name}: expected {dim1} columns, got shape {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: expected {numel} elements, got {t.numel()}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name}: holds {t.numel()} elements, the call needs {min_numel}")
    return t.device


def _need_current(dev):
    """Kernels launch on the current device: the tensors must live there."""
    cur = torch.cuda.current_device()
    if dev.index is not None and dev.index != cur:
        raise ValueError(f"tensors on {dev}, but the current device is cuda:{cur}")


def _need_dims(**dims):
    for name, v in dims.items():
        if int(v) != v or v < 0:
            raise ValueError(f"{name} must be a non-negative integer, got {v!r}")


def _packed(fmt, rows, k):
    """Bytes of a packed rows x k matrix; 0 for a shape the format cannot
    hold (the library itself rejects those with QBLK_ERR_SHAPE/FORMAT before
    touching memory)."""
    return packed_bytes(fmt, rows, k)


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
    dev = _need(w, "w", _FLOAT_IN, ndim=2)
    rows, k = w.shape
    nbytes = _packed(fmt, rows, k)
    if out is None:
        out = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=w.device)
    _need(out, "out", (torch.uint8,), min_numel=nbytes, device=dev)
    _need_current(dev)
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
    _need_dims(rows=rows, k=k)
    dev = _need(blocks, "blocks", (torch.uint8,), min_numel=_packed(fmt, rows, k))
    if out is None:
        out = torch.empty((rows, k), dtype=dtype, device=blocks.device)
    _need(out, "out", _FLOAT_IN, min_numel=rows * k, device=dev)
    _need_current(dev)
    _check(_lib.qblk_dequant(fmt, _ptr(blocks), rows, k, _ptr(out), _dtype(out), _stream(stream)),
           "qblk_dequant")
    return out


def gemv(blocks, fmt, m, k, x, out=None, stream=None):
    _need_dims(m=m, k=k)
    dev = _need(x, "x", _FLOAT_IN, numel=k)
    _need(blocks, "blocks", (torch.uint8,), min_numel=_packed(fmt, m, k), device=dev)
    if out is None:
        out = torch.empty(m, dtype=torch.float32, device=x.device)
    _need(out, "out", (torch.float32,), min_numel=m, device=dev)
    _need_current(dev)
    _check(_lib.qblk_gemv(fmt, _ptr(blocks), m, k, _ptr(x), _dtype(x), _ptr(out), _stream(stream)),
           "qblk_gemv")
    return out


class _GemvItem(C.Structure):
    """qblk_gemv_item_t"""
    _fields_ = [("blocks", C.c_void_p), ("m", C.c_int64), ("x", C.c_void_p), ("y", C.c_void_p)]


GEMV_BATCH_MAX = 32


def gemv_batch(fmt, k, products, outs=None, stream=None):
    """Several batch-1 products of equal k and x type in one call:
    products = [(blocks, m, x), ...]; returns [y, ...] (fp32, m each)."""
    _need_dims(k=k)
    if len(products) > GEMV_BATCH_MAX:
        raise ValueError(f"at most {GEMV_BATCH_MAX} products per call, got {len(products)}")
    if outs is not None and len(outs) != len(products):
        raise ValueError("outs: one output per product")
    items = (_GemvItem * max(1, len(products)))()
    ys, dev, xt = [], None, None
    for i, (blocks, m, x) in enumerate(products):
        _need_dims(m=m)
        dev = _need(x, f"x[{i}]", _FLOAT_IN, numel=k, device=dev)
        if xt is None:
            xt = x.dtype
        elif x.dtype != xt:
            raise TypeError(f"x[{i}]: element type {x.dtype}, the batch's first is {xt}")
        _need(blocks, f"blocks[{i}]", (torch.uint8,), min_numel=_packed(fmt, m, k), device=dev)
        y = outs[i] if outs is not None else torch.empty(m, dtype=torch.float32, device=x.device)
        _need(y, f"out[{i}]", (torch.float32,), min_numel=m, device=dev)
        items[i] = _GemvItem(_ptr(blocks).value, m, _ptr(x).value, _ptr(y).value)
        ys.append(y)
    if not products:
        return ys
    _need_current(dev)
    _check(_lib.qblk_gemv_batch(fmt, k, _DT[xt], C.cast(items, C.c_void_p), len(products), _stream(stream)),
           "qblk_gemv_batch")
    return ys


def gemm(blocks, fmt, m, k, X, out=None, stream=None):
    _need_dims(m=m, k=k)
    dev = _need(X, "X", _FLOAT_IN, ndim=2, dim1=k)
    n = X.shape[0]
    _need(blocks, "blocks", (torch.uint8,), min_numel=_packed(fmt, m, k), device=dev)
    if out is None:
        out = torch.empty((n, m), dtype=torch.float32, device=X.device)
    _need(out, "out", (torch.float32,), min_numel=n * m, device=dev)
    _need_current(dev)
    _check(_lib.qblk_gemm(fmt, _ptr(blocks), m, k, _ptr(X), _dtype(X), n, _ptr(out),
                          _stream(stream)), "qblk_gemm")
    return out


def quantize_act_i8(x, out=None, scale=None, stream=None):
    """8-bit activations: (n, k) f32/f16/bf16 -> (int8 codes (n, k), fp32 scales (n,))."""
    dev = _need(x, "x", _FLOAT_IN, ndim=2)
    n, k = x.shape
    if out is None:
        out = torch.empty((n, k), dtype=torch.int8, device=x.device)
    if scale is None:
        scale = torch.empty(n, dtype=torch.float32, device=x.device)
    _need(out, "out", (torch.int8,), min_numel=n * k, device=dev)
    _need(scale, "scale", (torch.float32,), min_numel=n, device=dev)
    _need_current(dev)
    _check(_lib.qblk_quantize_act_i8(_ptr(x), _dtype(x), n, k, _ptr(out), _ptr(scale), _stream(stream)),
           "qblk_quantize_act_i8")
    return out, scale


def gemm_w4a8(blocks, m, k, xq, scale, out=None, stream=None):
    """Y (n, m) fp32 = the W4A8 product of QBLK_W4G128 blocks and int8 activations."""
    _need_dims(m=m, k=k)
    dev = _need(xq, "xq", (torch.int8,), ndim=2, dim1=k)
    n = xq.shape[0]
    _need(scale, "scale", (torch.float32,), min_numel=n, device=dev)
    _need(blocks, "blocks", (torch.uint8,), min_numel=_packed(W4G128, m, k), device=dev)
    if out is None:
        out = torch.empty((n, m), dtype=torch.float32, device=xq.device)
    _need(out, "out", (torch.float32,), min_numel=n * m, device=dev)
    _need_current(dev)
    _check(_lib.qblk_gemm_w4a8(_ptr(blocks), m, k, _ptr(xq), _ptr(scale), n, _ptr(out), _stream(stream)),
           "qblk_gemm_w4a8")
    return out
