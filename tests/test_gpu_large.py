"""Calls past the size one launch can hold (GPU, through the C ABI).

A dispatch counts its threads in 32 bits per grid dimension.  The batch-1
products therefore run at most 2^24 rows per launch, and the activation
quantizer (one workgroup of 256 threads per row) at most
(2^32 - 1) / 256 = 16,777,215 rows per launch; longer calls run as several
launches in stream order.  These tests make calls just past those sizes, on
random packed matrices built on the GPU (random code bytes, finite fp16
scales), and check sampled rows, the rows on both sides of every piece
boundary and the last rows against the oracle.
"""
import numpy as np
import pytest

import oracle as O

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-5
GEMV_ROWS_PER_LAUNCH = 1 << 24
ACT_ROWS_PER_LAUNCH = (2**32 - 1) // 256
ROW_BYTES = {O.Q4_0: lambda k: k // 32 * 18, O.SB4: lambda k: k // 256 * 138}


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_block_quant_amd as q
    return q


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def random_blocks(fmt, m, k, seed):
    """A packed m x k matrix of random code bytes whose fp16 scales are
    finite and positive (bits 0x1400..0x2bff: 2^-10 .. 2^-4)."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    nb = O.packed_bytes(fmt, m, k)
    b = torch.randint(0, 256, (nb,), dtype=torch.uint8, device="cuda", generator=g)

    def scales(count):
        bits = torch.randint(0x1400, 0x2C00, (count,), dtype=torch.int32, device="cuda", generator=g)
        return bits.to(torch.int16).view(torch.uint8).view(count, 2)

    if fmt in (O.Q4_0, O.SB4):
        per = 18 if fmt == O.Q4_0 else 138
        v = b.view(-1, per)
        v[:, 0:2] = scales(v.shape[0])
    else:  # W4G128: codes of every row, then one fp16 scale per row and group
        sc = b[m * k // 2:].view(-1, 2)
        sc.copy_(scales(sc.shape[0]))
    return b


def rows_to_check(m, boundaries, seed, count=600):
    r = np.random.default_rng(seed).choice(m, size=count, replace=False)
    edges = [e + d for e in boundaries for d in (-2, -1, 0, 1)] + [0, m - 2, m - 1]
    return np.unique(np.concatenate([r, [e for e in edges if 0 <= e < m]]))


def check(y, y_ref, bound, what):
    err = np.abs(y.astype(np.float64) - y_ref)
    ok = err <= TOL * bound
    assert ok.all(), f"{what}: {np.count_nonzero(~ok)} outputs out of tolerance"


def oracle_rows(fmt, blocks, k, rows, x):
    """Oracle products of the listed rows (their blocks gathered into a small matrix)."""
    rb = ROW_BYTES[fmt](k)
    sub = host(blocks.view(-1, rb)[torch.from_numpy(rows).cuda()])
    return O.gemv(fmt, sub.reshape(-1), len(rows), k, x)


@pytest.mark.parametrize("fmt,k", [(O.Q4_0, 32), (O.SB4, 256)], ids=["q4_0-k32", "sb4-k256"])
@pytest.mark.parametrize("xt", [torch.float16, torch.float32], ids=["f16", "f32"])
def test_gemv_rows_in_pieces(q, fmt, k, xt):
    m = GEMV_ROWS_PER_LAUNCH + 5  # two launches: 2^24 rows, then 5
    blocks = random_blocks(fmt, m, k, 301 + fmt)
    x = torch.from_numpy(np.random.default_rng(302).standard_normal(k).astype(np.float32)).cuda().to(xt)
    y = host(q.gemv(blocks, fmt, m, k, x))
    rows = rows_to_check(m, [GEMV_ROWS_PER_LAUNCH], 303)
    y_ref, bound = oracle_rows(fmt, blocks, k, rows, host(x.float()).astype(np.float64))
    check(y[rows], y_ref, bound, f"gemv fmt={fmt} m={m}")
    del blocks


def test_gemv_batch_past_one_launch(q):
    # two products whose rows together pass one launch: one launch per product
    k, m = 256, GEMV_ROWS_PER_LAUNCH // 2 + 3
    x = torch.from_numpy(np.random.default_rng(311).standard_normal(k).astype(np.float32)).cuda().half()
    mats = [random_blocks(O.SB4, m, k, 312 + i) for i in range(2)]
    ys = q.gemv_batch(q.SB4, k, [(b, m, x) for b in mats])
    xv = host(x.float()).astype(np.float64)
    for i, (b, y) in enumerate(zip(mats, ys)):
        rows = rows_to_check(m, [], 313 + i, count=300)
        y_ref, bound = oracle_rows(O.SB4, b, k, rows, xv)
        check(host(y)[rows], y_ref, bound, f"gemv_batch item {i}")


def test_gemv_w4a8_rows_in_pieces(q):
    m, k = GEMV_ROWS_PER_LAUNCH + 5, 128
    blocks = random_blocks(O.W4G128, m, k, 321)
    x = torch.from_numpy(np.random.default_rng(322).standard_normal((1, k)).astype(np.float32)).cuda()
    xq, s = q.quantize_act_i8(x)
    y = host(q.gemm_w4a8(blocks, m, k, xq, s))
    rows = rows_to_check(m, [GEMV_ROWS_PER_LAUNCH], 323)
    ri = torch.from_numpy(rows).cuda()
    codes = host(blocks[: m * k // 2].view(m, k // 2)[ri])
    scales = host(blocks[m * k // 2:].view(m, 2 * (k // 128))[ri])
    sub = np.concatenate([codes.reshape(-1), scales.reshape(-1)])
    y_ref, bound = O.gemm_w4a8(sub, len(rows), k, host(xq), host(s))
    check(y[0, rows], y_ref[0], bound[0], f"w4a8 gemv m={m}")
    del blocks


def test_quantize_act_i8_rows_in_pieces(q):
    n, k = ACT_ROWS_PER_LAUNCH + 3, 8  # two launches: 16,777,215 rows, then 3
    g = torch.Generator(device="cuda").manual_seed(331)
    x = torch.randn((n, k), device="cuda", generator=g)
    xq, s = q.quantize_act_i8(x)
    rows = rows_to_check(n, [ACT_ROWS_PER_LAUNCH], 332, count=2000)
    ri = torch.from_numpy(rows).cuda()
    xq_ref, s_ref = O.quantize_act_i8(host(x[ri]))
    assert np.array_equal(host(xq[ri]), xq_ref)
    assert np.array_equal(host(s[ri]).view(np.uint32), s_ref.view(np.uint32))
