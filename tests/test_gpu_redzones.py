"""Out-of-bounds checks of every entry point on the GPU (through the C ABI).

Each buffer a call receives sits in the middle of a larger allocation whose
4 KiB margins on both sides hold a poison pattern (0xFF bytes: NaN in every
float type, NaN scales in every block format).  After the call the margins
must be unchanged (no write outside the buffer), and the results must equal
those of the same call on plain tensors (a read of the poison that reaches a
result would show as a NaN or a changed value).  Shapes cover every kernel
the dispatch picks, with ragged row, column and token tails.
"""
import numpy as np
import pytest

import workloads as WL

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MARGIN = 4096
POISON = 0xFF
Q4_0, SB4, SB4_AFFINE, Q4_K, W4G128 = 0, 1, 2, 3, 4  # qblk_format_t


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_block_quant_amd as q
    assert (q.Q4_0, q.SB4, q.SB4_AFFINE, q.Q4_K, q.W4G128) == (Q4_0, SB4, SB4_AFFINE, Q4_K, W4G128)
    return q


class Padded:
    """A tensor of `shape`/`dtype` inside a poisoned allocation."""

    def __init__(self, shape, dtype, init=None):
        self.nbytes = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.whole = torch.full((self.nbytes + 2 * MARGIN,), POISON, dtype=torch.uint8, device="cuda")
        inner = self.whole[MARGIN:MARGIN + self.nbytes]
        self.t = inner.view(dtype).view(shape) if self.nbytes else torch.empty(shape, dtype=dtype, device="cuda")
        if init is not None:
            self.t.copy_(init)

    def margins_intact(self):
        torch.cuda.synchronize()
        w = self.whole.cpu().numpy()
        return bool(np.all(w[:MARGIN] == POISON) and np.all(w[MARGIN + self.nbytes:] == POISON))


def padded_like(t):
    return Padded(tuple(t.shape), t.dtype, t)


def same(a, b, exact=True):
    a, b = a.detach().cpu(), b.detach().cpu()
    if exact:
        return torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                           b.view(torch.uint8) if b.dtype != torch.uint8 else b)
    a, b = a.double().numpy(), b.double().numpy()
    if not np.all(np.isfinite(a)):
        return False
    scale = max(1e-30, float(np.max(np.abs(b))))
    return float(np.max(np.abs(a - b))) <= 1e-5 * scale


def weights(rows, k, seed):
    return torch.from_numpy(WL.normal((rows, k), 0.02, seed)).cuda()


FLOAT_TYPES = [torch.float32, torch.float16, torch.bfloat16]


@pytest.mark.parametrize("fmt,rows,k", [(Q4_0, 37, 96), (SB4, 37, 512), (SB4_AFFINE, 37, 512),
                                        (Q4_K, 37, 512), (Q4_0, 300, 4096), (SB4, 300, 4096)])
@pytest.mark.parametrize("dtype", FLOAT_TYPES, ids=["f32", "f16", "bf16"])
def test_quantize_dequant_margins(q, fmt, rows, k, dtype):
    w = weights(rows, k, 201).to(dtype)
    ref = q.quantize(w, fmt)
    pw = padded_like(w)
    pb = Padded((q.packed_bytes(fmt, rows, k),), torch.uint8)
    out = q.quantize(pw.t, fmt, out=pb.t)
    assert pw.margins_intact() and pb.margins_intact()
    assert same(out, ref)
    for ot in FLOAT_TYPES:
        dref = q.dequant(ref, fmt, rows, k, dtype=ot)
        po = Padded((rows, k), ot)
        q.dequant(pb.t, fmt, rows, k, out=po.t)
        assert pb.margins_intact() and po.margins_intact()
        assert same(po.t, dref)


def test_quantize_q4_0_listing_and_w4g128_margins(q):
    w = weights(29, 384, 202)
    for fmt, ref_mode in ((Q4_0, True), (W4G128, False)):
        ref = q.quantize(w, fmt, ref=ref_mode)
        pw = padded_like(w)
        pb = Padded((q.packed_bytes(fmt, 29, 384),), torch.uint8)
        q.quantize(pw.t, fmt, out=pb.t, ref=ref_mode)
        assert pw.margins_intact() and pb.margins_intact()
        assert same(pb.t, ref)


@pytest.mark.parametrize("fmt,m,k", [(Q4_0, 37, 96), (Q4_0, 4096, 4096), (SB4, 37, 512),
                                     (SB4, 11008, 4096), (SB4, 4096, 11008), (SB4_AFFINE, 300, 4096),
                                     (Q4_K, 300, 4096), (SB4, 70, 13056)])
@pytest.mark.parametrize("xt", FLOAT_TYPES, ids=["f32", "f16", "bf16"])
def test_gemv_margins(q, fmt, m, k, xt):
    blocks = q.quantize(weights(m, k, 203), fmt)
    x = torch.from_numpy(WL.normal((k,), 1.0, 204)).cuda().to(xt)
    ref = q.gemv(blocks, fmt, m, k, x)
    pb, px, py = padded_like(blocks), padded_like(x), Padded((m,), torch.float32)
    q.gemv(pb.t, fmt, m, k, px.t, out=py.t)
    assert pb.margins_intact() and px.margins_intact() and py.margins_intact()
    assert same(py.t, ref)


@pytest.mark.parametrize("fmt", [Q4_0, SB4, SB4_AFFINE, Q4_K])
@pytest.mark.parametrize("k,xt", [(4096, torch.float16), (11008, torch.float16), (2304, torch.float32)],
                         ids=["4096-f16", "11008-f16", "2304-f32"])
def test_gemv_batch_margins(q, fmt, k, xt):
    ms = [300, 37, 4096, 1]
    prods, refs, pads = [], [], []
    for i, m in enumerate(ms):
        blocks = q.quantize(weights(m, k, 209 + i), fmt)
        x = torch.from_numpy(WL.normal((k,), 1.0, 213 + i)).cuda().to(xt)
        refs.append(q.gemv(blocks, fmt, m, k, x))
        pb, px, py = padded_like(blocks), padded_like(x), Padded((m,), torch.float32)
        pads += [pb, px, py]
        prods.append((pb.t, m, px.t))
    q.gemv_batch(fmt, k, prods, outs=[p.t for p in pads[2::3]])
    assert all(p.margins_intact() for p in pads)
    for py, ref in zip(pads[2::3], refs):
        assert same(py.t, ref, exact=False)


@pytest.mark.parametrize("fmt", [Q4_0, SB4, SB4_AFFINE, Q4_K])
@pytest.mark.parametrize("m,k,n", [(150, 2304, 1), (150, 2304, 16), (150, 2304, 40), (150, 2304, 100),
                                   (150, 2304, 200), (40, 14336, 130), (2000, 1024, 300)])
def test_gemm_margins(q, fmt, m, k, n):
    blocks = q.quantize(weights(m, k, 205), fmt)
    X = torch.from_numpy(WL.normal((n, k), 1.0, 206)).cuda().to(torch.bfloat16)
    ref = q.gemm(blocks, fmt, m, k, X)
    pb, px, py = padded_like(blocks), padded_like(X), Padded((n, m), torch.float32)
    q.gemm(pb.t, fmt, m, k, px.t, out=py.t)
    assert pb.margins_intact() and px.margins_intact() and py.margins_intact()
    assert same(py.t, ref, exact=False)


@pytest.mark.parametrize("n,k", [(1, 4096), (7, 384), (300, 2048)])
@pytest.mark.parametrize("xt", FLOAT_TYPES, ids=["f32", "f16", "bf16"])
def test_w4a8_margins(q, n, k, xt):
    m = 150
    blocks = q.quantize(weights(m, k, 207), W4G128)
    x = torch.from_numpy(WL.normal((n, k), 1.0, 208)).cuda().to(xt)
    xq_ref, s_ref = q.quantize_act_i8(x)
    px, pq, ps = padded_like(x), Padded((n, k), torch.int8), Padded((n,), torch.float32)
    q.quantize_act_i8(px.t, out=pq.t, scale=ps.t)
    assert px.margins_intact() and pq.margins_intact() and ps.margins_intact()
    assert same(pq.t, xq_ref) and same(ps.t, s_ref)
    ref = q.gemm_w4a8(blocks, m, k, xq_ref, s_ref)
    pb, py = padded_like(blocks), Padded((n, m), torch.float32)
    q.gemm_w4a8(pb.t, m, k, pq.t, ps.t, out=py.t)
    assert pb.margins_intact() and pq.margins_intact() and ps.margins_intact() and py.margins_intact()
    assert same(py.t, ref, exact=False)
