"""The Python binding's argument checks (CPU only, no kernel is launched).

The C ABI receives raw pointers and cannot see tensor extents, so the binding
must reject, before any call into the library, every tensor that is not on
the GPU, not contiguous, of the wrong element type, of the wrong shape or too
small for the call.  Each case below must raise and must not reach a compute
entry point: the library handle is replaced by a stand-in that records calls
(geometry queries are passed through to the real library)."""
import os

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "bit_block_quant_amd", "libqblk.so")
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libqblk.so not built")


class FakeGpuTensor:
    """Enough of a torch tensor for the checks: a GPU tensor of a given shape,
    element type, contiguity and device, with no storage behind it."""

    def __init__(self, shape, dtype, contiguous=True, index=0):
        self.shape = tuple(shape)
        self.dtype = dtype
        self.is_cuda = True
        self.device = torch.device("cuda", index)
        self._contiguous = contiguous

    def is_contiguous(self):
        return self._contiguous

    def dim(self):
        return len(self.shape)

    def numel(self):
        n = 1
        for d in self.shape:
            n *= d
        return n


class RecordingLib:
    """Stands in for the ctypes library: geometry passes through, any compute
    entry point is recorded (and would fail the test)."""

    GEOMETRY = ("qblk_packed_bytes", "qblk_block_bytes", "qblk_block_elems", "qblk_status_string")

    def __init__(self, real):
        self.real = real
        self.calls = []

    def __getattr__(self, name):
        if name in self.GEOMETRY:
            return getattr(self.real, name)

        def record(*a):
            self.calls.append(name)
            return 0
        return record


@pytest.fixture()
def q(monkeypatch):
    import bit_block_quant_amd as q
    rec = RecordingLib(q._lib)
    monkeypatch.setattr(q, "_lib", rec)
    yield q
    assert rec.calls == [], f"a compute entry point was reached: {rec.calls}"


F32, F16, BF16, U8, I8 = torch.float32, torch.float16, torch.bfloat16, torch.uint8, torch.int8
M, K = 64, 512  # 2 super-blocks per row


def sb4_blocks(q, rows=M, k=K, shrink=0):
    return FakeGpuTensor((q.packed_bytes(q.SB4, rows, k) - shrink,), U8)


def test_cpu_tensors_rejected(q):
    w = torch.zeros((M, K), dtype=F32)
    with pytest.raises(ValueError, match="GPU tensor"):
        q.quantize(w, q.SB4)
    with pytest.raises(ValueError, match="GPU tensor"):
        q.gemv(sb4_blocks(q), q.SB4, M, K, torch.zeros(K, dtype=F16))
    with pytest.raises(ValueError, match="GPU tensor"):
        q.gemm(sb4_blocks(q), q.SB4, M, K, torch.zeros((4, K), dtype=BF16))
    with pytest.raises(ValueError, match="GPU tensor"):
        q.quantize_act_i8(torch.zeros((4, K), dtype=F16))


def test_quantize_checks(q):
    with pytest.raises(ValueError, match="contiguous"):  # a transposed view
        q.quantize(FakeGpuTensor((M, K), F32, contiguous=False), q.SB4)
    with pytest.raises(ValueError, match="dimensions"):
        q.quantize(FakeGpuTensor((M * K,), F32), q.SB4)
    with pytest.raises(TypeError, match="element type"):
        q.quantize(FakeGpuTensor((M, K), torch.int32), q.SB4)
    short = FakeGpuTensor((q.packed_bytes(q.SB4, M, K) - 1,), U8)
    with pytest.raises(ValueError, match="needs"):
        q.quantize(FakeGpuTensor((M, K), F32), q.SB4, out=short)
    with pytest.raises(TypeError, match="element type"):
        q.quantize(FakeGpuTensor((M, K), F32), q.SB4, out=FakeGpuTensor((10 ** 6,), I8))


def test_dequant_checks(q):
    with pytest.raises(ValueError, match="needs"):
        q.dequant(sb4_blocks(q, shrink=1), q.SB4, M, K, out=FakeGpuTensor((M, K), F32))
    with pytest.raises(ValueError, match="needs"):
        q.dequant(sb4_blocks(q), q.SB4, M, K, out=FakeGpuTensor((M, K - 1), F32))
    with pytest.raises(ValueError, match="non-negative"):
        q.dequant(sb4_blocks(q), q.SB4, -1, K, out=FakeGpuTensor((M, K), F32))


def test_gemv_checks(q):
    x = FakeGpuTensor((K,), F16)
    with pytest.raises(ValueError, match="expected 512 elements"):
        q.gemv(sb4_blocks(q), q.SB4, M, K, FakeGpuTensor((K - 32,), F16))
    with pytest.raises(ValueError, match="needs"):
        q.gemv(sb4_blocks(q, shrink=1), q.SB4, M, K, x)
    with pytest.raises(ValueError, match="needs"):
        q.gemv(sb4_blocks(q), q.SB4, M, K, x, out=FakeGpuTensor((M - 1,), F32))
    with pytest.raises(TypeError, match="element type"):
        q.gemv(sb4_blocks(q), q.SB4, M, K, x, out=FakeGpuTensor((M,), F16))
    with pytest.raises(ValueError, match="contiguous"):
        q.gemv(sb4_blocks(q), q.SB4, M, K, FakeGpuTensor((K,), F16, contiguous=False))
    with pytest.raises(ValueError, match="other arguments"):  # blocks on another GPU than x
        q.gemv(FakeGpuTensor((q.packed_bytes(q.SB4, M, K),), U8, index=1), q.SB4, M, K, x)


def test_gemm_checks(q):
    with pytest.raises(ValueError, match="columns"):  # X must be n x k, token-major
        q.gemm(sb4_blocks(q), q.SB4, M, K, FakeGpuTensor((K, 4), BF16))
    with pytest.raises(ValueError, match="dimensions"):
        q.gemm(sb4_blocks(q), q.SB4, M, K, FakeGpuTensor((4 * K,), BF16))
    with pytest.raises(ValueError, match="contiguous"):  # a transposed view of a k x n matrix
        q.gemm(sb4_blocks(q), q.SB4, M, K, FakeGpuTensor((4, K), BF16, contiguous=False))
    with pytest.raises(ValueError, match="needs"):
        q.gemm(sb4_blocks(q), q.SB4, M, K, FakeGpuTensor((4, K), BF16), out=FakeGpuTensor((4, M - 1), F32))
    with pytest.raises(ValueError, match="needs"):
        q.gemm(sb4_blocks(q, shrink=1), q.SB4, M, K, FakeGpuTensor((4, K), BF16))


def test_w4a8_checks(q):
    blocks = FakeGpuTensor((q.packed_bytes(q.W4G128, M, K),), U8)
    xq = FakeGpuTensor((4, K), I8)
    with pytest.raises(ValueError, match="needs"):
        q.gemm_w4a8(blocks, M, K, xq, FakeGpuTensor((3,), F32))
    with pytest.raises(TypeError, match="element type"):
        q.gemm_w4a8(blocks, M, K, FakeGpuTensor((4, K), U8), FakeGpuTensor((4,), F32))
    with pytest.raises(ValueError, match="columns"):
        q.gemm_w4a8(blocks, M, K, FakeGpuTensor((4, K // 2), I8), FakeGpuTensor((4,), F32))
    with pytest.raises(ValueError, match="needs"):
        q.gemm_w4a8(FakeGpuTensor((q.packed_bytes(q.W4G128, M, K) - 1,), U8), M, K, xq, FakeGpuTensor((4,), F32))
    with pytest.raises(ValueError, match="needs"):
        q.quantize_act_i8(FakeGpuTensor((4, K), F16), out=FakeGpuTensor((4, K - 1), I8),
                          scale=FakeGpuTensor((4,), F32))
    with pytest.raises(ValueError, match="needs"):
        q.quantize_act_i8(FakeGpuTensor((4, K), F16), out=FakeGpuTensor((4, K), I8), scale=FakeGpuTensor((3,), F32))
