"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/qblk.h declares, reports the format geometry, and
rejects bad arguments before any HIP call."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qblk.h")


def _declared():
    src = open(HEADER, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qblk_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def q():
    import bit_block_quant_amd as q
    return q


def test_header_declares_the_entry_points():
    names = _declared()
    for f in ("qblk_quantize_q4_0", "qblk_quantize_sb4", "qblk_quantize_q4_k", "qblk_dequant", "qblk_gemv",
              "qblk_gemm"):
        assert f in names


def test_library_exports_every_declared_symbol(q):
    lib = C.CDLL(q.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    assert set(_declared()) == set(q.EXPORTS)


def test_geometry(q):
    assert [q.block_bytes(f) for f in (q.Q4_0, q.SB4, q.SB4_AFFINE, q.Q4_K)] == [18, 138, 148, 144]
    assert [q.block_elems(f) for f in (q.Q4_0, q.SB4, q.SB4_AFFINE, q.Q4_K)] == [32, 256, 256, 256]
    assert q.packed_bytes(q.Q4_K, 11008, 4096) == 11008 * 16 * 144
    assert q.block_bytes(q.W4G128) == 66 and q.block_elems(q.W4G128) == 128
    assert q.packed_bytes(q.W4G128, 11008, 4096) == 11008 * 4096 // 2 + 11008 * 32 * 2
    assert q.packed_bytes(q.W4G128, 3, 192) == 0
    assert q.block_bytes(9) == 0 and q.block_elems(9) == 0
    assert q.packed_bytes(q.SB4, 11008, 4096) == 24305664
    assert q.packed_bytes(q.Q4_0, 4096, 4096) == 9437184
    assert q.packed_bytes(q.SB4_AFFINE, 4096, 11008) == 4096 * 43 * 148
    assert q.packed_bytes(q.SB4, 3, 100) == 0  # k not a multiple of 256
    assert q.packed_bytes(q.Q4_0, -1, 32) == 0
    assert q.version().count(".") == 2


def test_status_strings(q):
    lib = q.lib()
    for st in range(8):
        assert lib.qblk_status_string(st)
    assert lib.qblk_status_string(99) == b"unknown status"


# Validation happens on the host before any launch.  Fake but 16-byte-aligned
# addresses are fine: a rejected call never dereferences them.
A, B, Y = C.c_void_p(0x10000), C.c_void_p(0x20000), C.c_void_p(0x30000)
MIS = C.c_void_p(0x10002)
NUL = C.c_void_p(0)
S = C.c_void_p(0)


def test_argument_errors(q):
    L = q.lib()
    # shapes
    assert L.qblk_quantize_q4_0(A, 0, 4, 33, B, S) == 2
    assert L.qblk_quantize_sb4(A, 0, 4, 32, 0, B, S) == 2
    assert L.qblk_quantize_sb4(A, 0, -1, 256, 1, B, S) == 2
    assert L.qblk_gemv(1, A, 1 << 31, 256, B, 1, Y, S) == 2
    assert L.qblk_gemm(1, A, 16, 256, B, 2, -1, Y, S) == 2
    assert L.qblk_gemm(1, A, (1 << 28) + 1, 256, B, 2, 2, Y, S) == 2  # at most 2^28 rows per product
    assert L.qblk_gemm_w4a8(A, (1 << 28) + 1, 128, B, Y, 2, Y, S) == 2
    # format / dtype
    assert L.qblk_dequant(7, A, 1, 256, B, 0, S) == 7
    assert L.qblk_gemv(1, A, 1, 256, B, 5, Y, S) == 3
    assert L.qblk_quantize_q4_0(A, 3, 1, 32, B, S) == 3
    assert L.qblk_quantize_q4_0_ref(A, 1, 1, 32, B, S) == 3
    assert L.qblk_quantize_q4_k(A, 3, 1, 256, B, S) == 3
    assert L.qblk_quantize_q4_k(A, 0, 1, 32, B, S) == 2
    assert L.qblk_quantize_q4_k(A, 0, 1, 256, MIS, S) == 4
    assert L.qblk_dequant(5, A, 1, 256, B, 0, S) == 7
    assert L.qblk_quantize_w4g128(A, 0, 1, 192, B, S) == 2
    assert L.qblk_quantize_w4g128(A, 4, 1, 128, B, S) == 3
    assert L.qblk_quantize_act_i8(A, 0, 2, 12, B, Y, S) == 2
    assert L.qblk_quantize_act_i8(A, 0, 2, 16, B, C.c_void_p(0x30001), S) == 4  # scales: 4-byte alignment
    assert L.qblk_gemm_w4a8(A, 4, 192, B, Y, 2, Y, S) == 2
    assert L.qblk_gemm_w4a8(A, 4, 128, B, NUL, 2, Y, S) == 1
    # group-128 weights multiply only 8-bit activations
    assert L.qblk_gemv(4, A, 4, 128, B, 1, Y, S) == 5
    assert L.qblk_gemm(4, A, 4, 256, B, 2, 4, Y, S) == 5
    # null and misaligned pointers
    assert L.qblk_quantize_q4_0(NUL, 0, 1, 32, B, S) == 1
    assert L.qblk_dequant(0, A, 1, 32, NUL, 0, S) == 1
    assert L.qblk_gemv(0, A, 1, 32, NUL, 1, Y, S) == 1
    assert L.qblk_gemv(0, A, 1, 32, B, 1, NUL, S) == 1
    assert L.qblk_gemv(1, MIS, 1, 256, B, 1, Y, S) == 4
    assert L.qblk_gemv(1, A, 1, 256, MIS, 1, Y, S) == 4
    assert L.qblk_quantize_sb4(A, 0, 1, 256, 0, MIS, S) == 4
    # GEMM support matrix: bf16 activations only; Q4_0 in whole 256-weight groups
    assert L.qblk_gemm(1, A, 16, 256, B, 1, 16, Y, S) == 5
    assert L.qblk_gemm(0, A, 16, 256, B, 0, 16, Y, S) == 5
    assert L.qblk_gemm(0, A, 16, 288, B, 2, 16, Y, S) == 5
    assert L.qblk_gemm(2, A, 16, 256, B, 1, 16, Y, S) == 5
    assert L.qblk_gemm(0, A, 16, 33, B, 2, 16, Y, S) == 2


def test_empty_calls_succeed_without_launch(q):
    L = q.lib()
    assert L.qblk_quantize_q4_0(NUL, 0, 0, 32, NUL, S) == 0
    assert L.qblk_quantize_sb4(NUL, 1, 5, 0, 1, NUL, S) == 0
    assert L.qblk_quantize_q4_k(NUL, 2, 0, 256, NUL, S) == 0
    assert L.qblk_quantize_act_i8(NUL, 1, 0, 256, NUL, NUL, S) == 0
    assert L.qblk_gemm_w4a8(NUL, 0, 256, NUL, NUL, 4, NUL, S) == 0
    assert L.qblk_dequant(2, NUL, 0, 256, NUL, 2, S) == 0
    assert L.qblk_gemv(1, NUL, 0, 256, NUL, 1, NUL, S) == 0
    assert L.qblk_gemm(1, NUL, 0, 256, NUL, 2, 8, NUL, S) == 0
    assert L.qblk_gemm(1, NUL, 8, 256, NUL, 2, 0, NUL, S) == 0


def test_deterministic_switch(q):
    assert q.deterministic() is False  # off at load
    try:
        q.set_deterministic(True)
        assert q.deterministic() is True
    finally:
        q.set_deterministic(False)
    assert q.deterministic() is False
