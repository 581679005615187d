"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Quantization and dequantization must match the oracle bit for bit; products
must satisfy |y - y_ref| <= 2e-5 * sum_k |W[i,k] x[k]| element by element
against the oracle's fp64 sums.  Inputs come from the seeded generators in
workloads/ (the configs' shapes and distributions) plus hand-made edge cases.
"""
import numpy as np
import pytest

import oracle as O
import workloads as WL

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 2e-5
FMTS = [O.Q4_0, O.SB4, O.SB4_AFFINE, O.Q4_K]
NAMES = {O.Q4_0: "q4_0", O.SB4: "sb4", O.SB4_AFFINE: "sb4a", O.Q4_K: "q4k"}


@pytest.fixture(scope="module")
def q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_block_quant_amd as q
    return q


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits):
    return dev(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def gpu_input(w, dtype):
    """Host f32 matrix -> (device tensor of dtype, host array the oracle reads)."""
    if dtype == "f32":
        return dev(w), w
    if dtype == "f16":
        h = w.astype(np.float16)
        return dev(h), h
    bits = WL.bf16_bits(w)
    return dev_bf16(bits), (bits, O.BF16)


def mixed_blocks(rows, k, seed):
    """Rows of several flavours (the edge cases of the formats)."""
    rng = np.random.default_rng(seed)
    w = np.empty((rows, k), np.float32)
    for r in range(rows):
        kind = r % 8
        if kind == 0:
            w[r] = rng.standard_normal(k) * 0.02
        elif kind == 1:
            w[r] = rng.standard_t(2, k) * 0.05
        elif kind == 2:  # exact half steps: ties of the rounding rule
            w[r] = (rng.integers(-15, 16, k) / 2.0) * 2.0 ** -6
            w[r, ::32] = 7 * 2.0 ** -6
        elif kind == 3:
            w[r] = rng.standard_normal(k) * 1e-6  # fp16-subnormal scales
        elif kind == 4:
            w[r] = 0.0
        elif kind == 5:  # constant sub-blocks and zeros
            w[r] = np.repeat(rng.standard_normal(k // 32), 32) * 0.01
            w[r, 64:128] = 0.0
        elif kind == 6:  # one outlier per 32 (the Q4_0 chapter's failure mode)
            w[r] = rng.uniform(-0.01, 0.01, k)
            w[r, 31::32] = 10.0
        else:
            w[r] = rng.standard_normal(k) * np.exp(rng.uniform(np.log(0.005), np.log(0.05)))
    return w


def near_ties(rows, k, seed):
    """Weights one fp32 ulp either side of a rounding tie of their block's quotient."""
    rng = np.random.default_rng(seed)
    w = (rng.integers(-14, 15, (rows, k)) / 2.0).astype(np.float32)
    w[:, ::32] = 7.0  # fixes each 32-block's scale at exactly 1.0
    flip = rng.integers(-1, 2, (rows, k)).astype(np.float32)
    w = np.where(flip > 0, np.nextafter(w, np.float32(np.inf)),
                 np.where(flip < 0, np.nextafter(w, np.float32(-np.inf)), w)).astype(np.float32)
    return w * np.float32(2.0 ** -8)


def affine_near_ties(rows, k, seed, dtype=np.float32):
    """Type 1 sub-blocks whose code quotients (w - a) / s sit on, or one ulp of
    the input type either side of, a half-integer: each 32-weight sub-block
    holds its min a and its max a + 15 s (s and a exact in fp16, so the stored
    offset and scale are a and s), and the other weights a + (c + 1/2) s,
    c = 0..14, each left alone or moved one ulp up or down."""
    rng = np.random.default_rng(seed)
    choices = [(-1.0, 0.125), (-0.25, 0.1875), (0.5, 3.0 / 256), (-3.0, 0.375), (-0.0625, 1.0 / 64)]
    w = np.empty((rows, k), dtype=np.float64)
    for r in range(rows):
        for j in range(k // 32):
            a, sc = choices[rng.integers(len(choices))]
            blk = a + (rng.integers(0, 15, 32) + 0.5) * sc
            blk[rng.integers(32)] = a
            blk[rng.integers(32)] = a + 15 * sc
            w[r, 32 * j:32 * j + 32] = blk
    w = w.astype(dtype)
    up, down = np.nextafter(w, dtype(np.inf)), np.nextafter(w, dtype(-np.inf))
    flip = rng.integers(-1, 2, w.shape)
    # keep each sub-block's extremes: only interior values move
    lo = w.reshape(rows, -1, 32).min(axis=2, keepdims=True)
    hi = w.reshape(rows, -1, 32).max(axis=2, keepdims=True)
    inner = ((w.reshape(rows, -1, 32) > lo) & (w.reshape(rows, -1, 32) < hi)).reshape(rows, k)
    w = np.where(inner & (flip > 0), up, np.where(inner & (flip < 0), down, w))
    return w.astype(dtype)


# ----------------------------------------------------------------- quantize
@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: NAMES[f])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_quantize_bit_exact(q, fmt, dtype):
    # 16 x 2304: 144 super-blocks or 1152 Q4_0 blocks; 3 x 768: 9 super-blocks
    # or 72 blocks, ragged tails of every quantizer's workgroup
    for w in (mixed_blocks(16, 2304, 1), near_ties(7, 2304, 2), mixed_blocks(3, 768, 3)):
        d, h = gpu_input(w, dtype)
        got = host(q.quantize(d, fmt))
        ref = O.quantize(fmt, h)
        assert got.shape == ref.shape
        assert np.array_equal(got, ref), f"first mismatch at byte {np.argmax(got != ref)}"


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_quantize_affine_near_ties(q, dtype):
    # quotients (w - a) / s on and one ulp around every half-integer code boundary
    w = affine_near_ties(9, 2304, 41, np.float32 if dtype == "f32" else np.float16)
    d = dev(w)
    got = host(q.quantize(d, q.SB4_AFFINE))
    ref = O.quantize(O.SB4_AFFINE, w)
    assert np.array_equal(got, ref), f"first mismatch at byte {np.argmax(got != ref)}"


def test_quantize_q4_0_listing_fixture_blocks(q):
    # the hand-derived blocks of the Q4_0 chapter's 4.4 quantizer (cap at 15,
    # the first extreme fixing the sign of d, codes from the fp32 reciprocal)
    import ast
    from test_oracle_pins import read_golden_raw
    g = read_golden_raw("q4_0_listing_cap_and_ties.txt")
    w = np.zeros((3, 32), dtype=np.float32)
    for r, name in enumerate(("cap", "first")):
        for i, v in ast.literal_eval(g[f"{name}_values"]).items():
            w[r, i] = v
    w[2, 0] = np.array([int(g["recip_e_bits"], 16)], np.uint32).view(np.float32)[0]
    w[2, 7] = np.array([int(g["recip_x_bits"], 16)], np.uint32).view(np.float32)[0]
    got = host(q.quantize(dev(w), q.Q4_0, ref=True))
    for r, name in enumerate(("cap", "first")):
        assert got[18 * r:18 * r + 18].tobytes() == bytes.fromhex(g[f"{name}_bytes"].replace(" ", ""))
    assert got[36 + 2 + 7] & 0x0F == int(g["recip_code_x"])
    assert np.array_equal(got, O.quantize_q4_0_ref(w))


def test_quantize_extreme_f16_inputs(q):
    w = np.full((2, 256), 65504.0, np.float16)
    w[0, ::2] = -65504.0
    w[1, :] = np.float16(6e-8)  # fp16 subnormal weights
    for fmt in FMTS:
        got = host(q.quantize(dev(w), fmt))
        assert np.array_equal(got, O.quantize(fmt, w)), NAMES[fmt]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_quantize_q4_k_one_sided_ranges_and_signed_zeros(q, dtype):
    # sub-blocks with no negative weight (min 0), none positive, negative
    # zeros only, a mix of +0 and -0, and single nonzero entries
    rng = np.random.default_rng(15)
    w = np.abs(rng.standard_normal((6, 2048)).astype(np.float32)) * 0.03
    w[1] = -w[1]
    w[2] = -0.0
    w[3, ::2] = -0.0
    w[3, 1::2] = 0.0
    w[4] = 0.0
    w[4, ::37] = -rng.uniform(0.01, 1.0, w[4, ::37].size)
    w[5, :1024] = -0.0
    d, h = gpu_input(w, dtype)
    got = host(q.quantize(d, q.Q4_K))
    assert np.array_equal(got, O.quantize_q4_k(h))


def test_quantize_q4_0_reference_mode(q):
    w = mixed_blocks(8, 4096, 3)
    vals = np.array([0.01 * (i - 15) / 15 for i in range(31)] + [10.0], np.float32)
    w[0, :32] = vals
    got = host(q.quantize(dev(w), q.Q4_0, ref=True))
    assert np.array_equal(got, O.quantize_q4_0_ref(w))


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: NAMES[f])
def test_quantize_full_size(q, fmt):
    w, _ = WL.sb4_decode("up") if fmt != O.Q4_0 else WL.q4_0_decode()
    got = host(q.quantize(dev(w), fmt))
    assert np.array_equal(got, O.quantize(fmt, w))


def test_quantize_stack_matrix_f16(q):
    for p in (0, 6):  # q (4096 x 4096) and down (4096 x 11008) of layer 0
        w, _ = WL.sb4a_stack_matrix(0, p)
        got = host(q.quantize(dev(w), q.SB4_AFFINE))
        assert np.array_equal(got, O.quantize_sb4(w, affine=True))


# ------------------------------------------------------------------ dequant
def random_blocks(fmt, nblk, seed):
    """Arbitrary bytes with finite fp16 scales."""
    rng = np.random.default_rng(seed)
    nb = O.block_bytes(fmt)
    b = rng.integers(0, 256, (nblk, nb), dtype=np.uint8)
    nscale = 2 if fmt in (O.SB4_AFFINE, O.Q4_K) else 1
    s = rng.integers(0, 0x7C00, (nblk, nscale)).astype(np.uint16)  # finite, incl. subnormal
    s |= (rng.integers(0, 2, (nblk, nscale)) << 15).astype(np.uint16)
    b[:, : 2 * nscale] = s.view(np.uint8).reshape(nblk, 2 * nscale)
    return b.reshape(-1)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: NAMES[f])
@pytest.mark.parametrize("ot", ["f32", "f16", "bf16"])
def test_dequant_bit_exact(q, fmt, ot):
    E = O.block_elems(fmt)
    rows, k = 5, E * 13  # ragged tail of the 2048-weight workgroups
    for blocks in (random_blocks(fmt, rows * k // E, 4),
                   O.quantize(fmt, mixed_blocks(rows, k, 5))):
        dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[ot]
        got = q.dequant(dev(blocks), fmt, rows, k, dt)
        ref = O.dequant(fmt, blocks, rows, k)
        if ot == "f32":
            assert np.array_equal(host(got).view(np.uint32), ref.view(np.uint32))
        elif ot == "f16":
            assert np.array_equal(host(got).view(np.uint16), ref.astype(np.float16).view(np.uint16))
        else:
            refb = torch.from_numpy(ref).to(torch.bfloat16).view(torch.int16).numpy()
            assert np.array_equal(host(got.view(torch.int16)), refb)


# --------------------------------------------------------------------- GEMV
def check_products(y, y_ref, bound, what):
    err = np.abs(y.astype(np.float64) - y_ref)
    ok = err <= TOL * bound
    assert ok.all(), f"{what}: {np.count_nonzero(~ok)} outputs out of tolerance, worst ratio {np.max(err / np.maximum(bound, 1e-300)):.3e}"
    zero = bound == 0
    assert np.all(y[zero] == 0), f"{what}: an all-zero product is not exactly 0"


def x_dev(x):
    if x.dtype == np.uint16:  # bf16 bits
        return dev_bf16(x), WL.bf16_values(x)
    return dev(x), x.astype(np.float64)


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: NAMES[f])
@pytest.mark.parametrize("xt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", [(1, 256), (37, 2304), (130, 11008), (1500, 1024)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_gemv_tolerance(q, fmt, xt, shape):
    m, k = shape
    w = mixed_blocks(m, k, 7 + m)
    blocks = O.quantize(fmt, w)
    xs = np.random.default_rng(8).standard_normal(k).astype(np.float32)
    x = {"f32": xs, "f16": xs.astype(np.float16), "bf16": WL.bf16_bits(xs)}[xt]
    xd, xr = x_dev(x)
    y = host(q.gemv(dev(blocks), fmt, m, k, xd))
    y_ref, bound = O.gemv(fmt, blocks, m, k, xr)
    check_products(y, y_ref, bound, f"{NAMES[fmt]} {xt} {shape}")


# x at the ends of its type's range: exact zeros, fp16 subnormals and
# +-65504, bf16/fp32 values near 1e+-30 and their smallest normals, mixed into
# N(0,1) values; zero units and whole zero rows of x's reach (y exactly 0 where
# the bound is 0).  Shapes that reach the per-wave, LDS-staged and generic
# kernels.
@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: NAMES[f])
@pytest.mark.parametrize("xt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", [(37, 2304), (4096, 4096), (300, 11008)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_gemv_extreme_x(q, fmt, xt, shape):
    m, k = shape
    w = mixed_blocks(m, k, 90 + m)
    blocks = O.quantize(fmt, w)
    rng = np.random.default_rng(91)
    xs = rng.standard_normal(k).astype(np.float32)
    idx = rng.permutation(k)
    if xt == "f16":
        big, small, tiny = 65504.0, 6.0e-8, 6.104e-5  # max, subnormal, smallest normal
    else:
        big, small, tiny = 1.0e30, 1.0e-30, 1.1754944e-38
    xs[idx[0:40:4]] = big
    xs[idx[1:40:4]] = -big
    xs[idx[2:40:4]] = small
    xs[idx[3:40:4]] = -tiny
    xs[64:96] = 0.0    # one whole unit of zeros
    xs[256:512] = 0.0  # one whole super-block of zeros
    x = xs if xt == "f32" else xs.astype(np.float16) if xt == "f16" else WL.bf16_bits(xs)
    xd, xr = x_dev(x)
    y = host(q.gemv(dev(blocks), fmt, m, k, xd))
    y_ref, bound = O.gemv(fmt, blocks, m, k, xr)
    check_products(y, y_ref, bound, f"{NAMES[fmt]} {xt} {shape} extreme x")


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: NAMES[f])
@pytest.mark.parametrize("k", [2304, 4096, 11008, 13056])
@pytest.mark.parametrize("xt", ["f16", "f32"])
def test_gemv_batch(q, fmt, k, xt):
    # several products in one call: ragged row counts (one empty), each its
    # own x; fp16 x up to 12288 weights per row shares one grid, the rest runs
    # per matrix -- every y against the oracle's product of its own matrix
    ms = [37, 4096, 0, 1000, 300]
    rng = np.random.default_rng(60 + k)
    cases = []
    for i, m in enumerate(ms):
        blocks = O.quantize(fmt, mixed_blocks(m, k, 61 + i)) if m else np.zeros(16, np.uint8)
        x = rng.standard_normal(k).astype(np.float16 if xt == "f16" else np.float32)
        cases.append((blocks, m, x))
    ys = q.gemv_batch(fmt, k, [(dev(b), m, dev(x)) for b, m, x in cases])
    for (blocks, m, x), y in zip(cases, ys):
        y = host(y)
        assert y.shape == (m,)
        if m:
            y_ref, bound = O.gemv(fmt, blocks, m, k, x.astype(np.float64))
            check_products(y, y_ref, bound, f"batch {NAMES[fmt]} {m}x{k} {xt}")


def test_gemv_batch_full(q):
    # the most products one call takes, row counts 1..~300 (the workgroup
    # ranges of 32 matrices in one grid, several matrices per workgroup round)
    k = 2304
    rng = np.random.default_rng(80)
    prods, cases = [], []
    for i in range(q.GEMV_BATCH_MAX):
        m = int(rng.integers(1, 300)) if i % 5 else 1
        blocks = O.quantize(O.SB4, mixed_blocks(m, k, 81 + i))
        x = rng.standard_normal(k).astype(np.float16)
        cases.append((blocks, m, x))
        prods.append((dev(blocks), m, dev(x)))
    ys = q.gemv_batch(O.SB4, k, prods)
    for (blocks, m, x), y in zip(cases, ys):
        y_ref, bound = O.gemv(O.SB4, blocks, m, k, x.astype(np.float64))
        check_products(host(y), y_ref, bound, f"full batch m={m}")
    with pytest.raises(ValueError):
        q.gemv_batch(O.SB4, k, prods + prods[:1])


def test_gemv_batch_matches_single_calls(q):
    # the headline shape inside a batch: each y agrees with the single call
    # (the batch's tiling follows its total rows, so the summation order may
    # differ: compared to 1e-4 of the largest output)
    k = 4096
    mats = [(11008, 70), (4096, 71), (4096, 72), (33, 73)]
    prods, singles = [], []
    for m, seed in mats:
        b = dev(O.quantize(O.SB4, mixed_blocks(m, k, seed)))
        x = dev(np.random.default_rng(seed).standard_normal(k).astype(np.float16))
        prods.append((b, m, x))
    ys = q.gemv_batch(O.SB4, k, prods)
    for (b, m, x), y in zip(prods, ys):
        y1 = host(q.gemv(b, O.SB4, m, k, x))
        assert np.allclose(host(y), y1, rtol=0, atol=1e-4 * max(1e-30, float(np.max(np.abs(y1)))))


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: NAMES[f])
@pytest.mark.parametrize("xt", ["f32", "f16"])
def test_gemv_unit_vector_is_a_column(q, fmt, xt):
    m, k = 70, 2048
    blocks = O.quantize(fmt, mixed_blocks(m, k, 9))
    W = O.dequant(fmt, blocks, m, k)
    bd = dev(blocks)
    for col in (0, 17, 1000, k - 1):
        x = np.zeros(k, np.float32 if xt == "f32" else np.float16)
        x[col] = 1
        y = host(q.gemv(bd, fmt, m, k, dev(x)))
        # exact values; a rebuilt weight of -0.0 (INT8 scale 0, code < 8) sums to +0.0
        assert np.array_equal(y, W[:, col]), col


def test_gemv_q4_0_small_config(q):
    w, x = WL.q4_0_small()
    b = q.quantize(dev(w), q.Q4_0)
    assert np.array_equal(host(b), O.quantize_q4_0(w))
    y = host(q.gemv(b, q.Q4_0, 256, 4096, dev(x)))
    y_ref, bound = O.gemv(O.Q4_0, O.quantize_q4_0(w), 256, 4096, x)
    check_products(y, y_ref, bound, "q4_0 256x4096 f32")


def test_gemv_q4_0_decode_config(q):
    w, x = WL.q4_0_decode()
    blocks = O.quantize_q4_0(w)
    y = host(q.gemv(dev(blocks), q.Q4_0, 4096, 4096, dev(x)))
    y_ref, bound = O.gemv(O.Q4_0, blocks, 4096, 4096, x.astype(np.float64))
    check_products(y, y_ref, bound, "q4_0 4096x4096 f16")


@pytest.mark.parametrize("shape", ["up", "down"])
def test_gemv_sb4_decode_config(q, shape):
    w, x = WL.sb4_decode(shape)
    m, k = w.shape
    blocks = O.quantize_sb4(w)
    y = host(q.gemv(dev(blocks), q.SB4, m, k, dev(x)))
    y_ref, bound = O.gemv(O.SB4, blocks, m, k, x.astype(np.float64))
    check_products(y, y_ref, bound, f"sb4 {m}x{k} f16")


def test_gemv_q4_k_decode_shape(q):
    w, x = WL.sb4_decode("up")
    m, k = w.shape
    blocks = O.quantize_q4_k(w)
    bd = q.quantize(dev(w), q.Q4_K)
    assert np.array_equal(host(bd), blocks)
    y = host(q.gemv(bd, q.Q4_K, m, k, dev(x)))
    y_ref, bound = O.gemv(O.Q4_K, blocks, m, k, x.astype(np.float64))
    check_products(y, y_ref, bound, f"q4k {m}x{k} f16")


def test_gemv_stack_matrices(q):
    for layer, p in ((0, 0), (0, 4), (31, 6)):
        w, x = WL.sb4a_stack_matrix(layer, p)
        m, k = w.shape
        blocks = O.quantize_sb4(w, affine=True)
        y = host(q.gemv(dev(blocks), q.SB4_AFFINE, m, k, dev(x)))
        y_ref, bound = O.gemv(O.SB4_AFFINE, blocks, m, k, x.astype(np.float64))
        check_products(y, y_ref, bound, f"sb4a layer {layer} proj {p}")


# fp16 x: every tiling of the up-front kernel (units of 32 weights per row S):
# S <= 64 one wave per row; S <= 128 two waves per row, one unit per lane
# (Type 0 and Q4_0 beyond 32 rows per CU: 16-wave workgroups with x staged
# in LDS before the weight loads, one wave per row, two units per lane, 3 row
# slots per wave -- from 33 rows per CU, where most waves repeat a row, to a
# last workgroup of 12 rows at 12300 x 4096; workgroups of up to 64 rows: 4
# slots of 16 rows, or 8 of 8 for the affine formats -- 14336 x 4096 with 56
# rows each; more rows per CU than that in equal rounds: 16385 x 4096 two
# rounds of 33 (the affine formats: two 8-wave workgroups per CU of 17 rows
# each), 12545 x 2048 (one wave per row) two of 25); S <= 256 two
# units per lane; S <= 384 three (Type 0 in 12-wave workgroups) -- with 1 to 8 row slots per wave (rows per
# CU 2 .. 64 and beyond, on 256 CUs), ragged halves (S = 33, 73), fewer
# rows than waves on every branch, and a one-unit row (S = 1).
GEMV_TILINGS = [(300, 2048), (5000, 2048), (11008, 2048), (2048, 4096), (6144, 4096), (8192, 4096), (8448, 4096),
                (8704, 4096), (10240, 4096), (12300, 4096), (12545, 2048), (14336, 4096), (16385, 4096),
                (500, 8192), (4096, 8192), (6200, 8192), (90, 1056), (700, 2336), (9000, 2336), (9000, 4064),
                (2560, 11008), (3990, 11264), (3, 1024), (3, 4096), (5, 8192), (2, 11264), (7, 32)]


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: NAMES[f])
@pytest.mark.parametrize("shape", GEMV_TILINGS, ids=lambda s: f"{s[0]}x{s[1]}")
def test_gemv_f16_tilings(q, fmt, shape):
    m, k = shape
    if fmt != q.Q4_0 and k % 256:
        pytest.skip("super-block formats need k % 256 == 0")
    rng = np.random.default_rng(m + k)
    w = (rng.standard_normal((m, k)) * 0.02).astype(np.float32)
    w[::7] *= 40.0  # rows of another magnitude
    x = rng.standard_normal(k).astype(np.float16)
    blocks = O.quantize(fmt, w)
    y = host(q.gemv(dev(blocks), fmt, m, k, dev(x)))
    y_ref, bound = O.gemv(fmt, blocks, m, k, x.astype(np.float64))
    check_products(y, y_ref, bound, f"{NAMES[fmt]} {m}x{k} f16")


def test_gemv_empty_k_writes_zeros(q):
    y = torch.full((33,), 7.0, device="cuda")
    q.gemv(torch.empty(0, dtype=torch.uint8, device="cuda"), q.SB4, 33, 0,
           torch.empty(0, dtype=torch.float16, device="cuda"), out=y)
    assert np.all(host(y) == 0)


def test_misaligned_pointer_is_rejected(q):
    b = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    x = torch.zeros(256, dtype=torch.float16, device="cuda")
    with pytest.raises(q.QblkError) as e:
        q.gemv(b[2:], q.SB4, 1, 256, x)
    assert e.value.status == 4


# --------------------------------------------------------------------- GEMM
# token counts chosen to reach every tiling: <= 16, <= 32, <= 64 and wide
# (one and two 128-token tiles), each with a ragged last tile
@pytest.mark.parametrize("n", [1, 5, 16, 24, 32, 33, 64, 100, 200])
def test_gemm_tolerance_small(q, n):
    m, k = 150, 2304
    w = mixed_blocks(m, k, 11)
    blocks = O.quantize_sb4(w)
    X = WL.bf16_bits(np.random.default_rng(12).standard_normal((n, k)).astype(np.float32))
    Y = host(q.gemm(dev(blocks), q.SB4, m, k, dev_bf16(X)))
    Y_ref, B = O.gemm(O.SB4, blocks, m, k, WL.bf16_values(X).astype(np.float64))
    check_products(Y, Y_ref, B, f"gemm n={n}")


# Activations of extreme spread and magnitude: within one token's super-block
# a largest |x| of 1.5 beside 2^-29 or 2^-30, a token scaled by 2^100, a value
# of 2^116, a super-block scaled by 2^-90, and whole tokens of zeros (exactly
# zero outputs), in a ragged shape (150 rows, 9 super-blocks).
@pytest.mark.parametrize("case", ["spread_2e-29", "spread_2e-30", "times_2e100", "value_2e116", "times_2e-90", "zero_tokens"])
def test_gemm_sb4_extreme_activations(q, case):
    m, k, n = 150, 2304, 11
    w = mixed_blocks(m, k, 21)
    blocks = O.quantize_sb4(w)
    Xf = np.random.default_rng(22).standard_normal((n, k)).astype(np.float32)
    if case == "spread_2e-29":      # 1.5 beside 2^-29
        Xf[3, 256:512] = 0.0
        Xf[3, 300], Xf[3, 301] = 1.5, 2.0 ** -29
    elif case == "spread_2e-30":   # 1.5 beside 2^-30
        Xf[3, 300], Xf[3, 301] = 1.5, 2.0 ** -30
    elif case == "times_2e100":    # a token's first super-block times 2^100
        Xf[5, :256] *= 2.0 ** 100
    elif case == "value_2e116":   # one value of 2^116
        Xf[5, :256] = 0.5
        Xf[5, 7] = 2.0 ** 116
    elif case == "times_2e-90":  # a super-block times 2^-90
        Xf[2, 1024:1280] *= 2.0 ** -90
    else:                      # whole tokens of zeros
        Xf[[0, 4, 10]] = 0.0
    X = WL.bf16_bits(Xf)
    Y = host(q.gemm(dev(blocks), q.SB4, m, k, dev_bf16(X)))
    Y_ref, B = O.gemm(O.SB4, blocks, m, k, WL.bf16_values(X).astype(np.float64))
    check_products(Y, Y_ref, B, f"gemm extreme activations {case}")


def gemm_fmt(q, name):
    """(library format id, oracle format id) for a format name."""
    return {"q4_0": (q.Q4_0, O.Q4_0), "sb4a": (q.SB4_AFFINE, O.SB4_AFFINE), "q4k": (q.Q4_K, O.Q4_K)}[name]


@pytest.mark.parametrize("fmt", ["q4_0", "sb4a", "q4k"])
@pytest.mark.parametrize("n", [1, 5, 16, 24, 32, 40, 64, 100])
def test_gemm_other_formats(q, fmt, n):
    # Q4_0 (scale per 32-block), Type 1 and Q4_K (scale and offset per sub-block)
    m, k = 150, 2304
    f, of = gemm_fmt(q, fmt)
    w = mixed_blocks(m, k, 21)
    blocks = O.quantize(of, w)
    X = WL.bf16_bits(np.random.default_rng(22).standard_normal((n, k)).astype(np.float32))
    Y = host(q.gemm(dev(blocks), f, m, k, dev_bf16(X)))
    Y_ref, B = O.gemm(of, blocks, m, k, WL.bf16_values(X).astype(np.float64))
    check_products(Y, Y_ref, B, f"gemm {fmt} n={n}")


@pytest.mark.parametrize("fmt", ["q4_0", "sb4a", "q4k"])
@pytest.mark.parametrize("n", [20, 130])
def test_gemm_other_formats_split_k(q, fmt, n):
    # long K with few rows: K is split over the grid and summed into Y
    m, k = 40, 14336
    f, of = gemm_fmt(q, fmt)
    w = mixed_blocks(m, k, 23)
    blocks = O.quantize(of, w)
    X = WL.bf16_bits(np.random.default_rng(24).standard_normal((n, k)).astype(np.float32))
    Y = host(q.gemm(dev(blocks), f, m, k, dev_bf16(X)))
    Y_ref, B = O.gemm(of, blocks, m, k, WL.bf16_values(X).astype(np.float64))
    check_products(Y, Y_ref, B, f"gemm {fmt} split-K")


@pytest.mark.parametrize("fmt", ["sb4a", "q4k"])
def test_gemm_affine_64_token_tiles_unsplit(q, fmt):
    # 12400 x 512, 200 tokens: 128-token tiles would fill under 3/4 of the
    # workgroup slots, so the affine formats take 64-token tiles (4 per column
    # of row tiles, the last one ragged), 388 tiles on 256 CUs: K not split
    m, k, n = 12400, 512, 200
    f, of = gemm_fmt(q, fmt)
    w = mixed_blocks(m, k, 25)
    blocks = O.quantize(of, w)
    X = WL.bf16_bits(np.random.default_rng(26).standard_normal((n, k)).astype(np.float32))
    Y = host(q.gemm(dev(blocks), f, m, k, dev_bf16(X)))
    rows = np.concatenate([np.random.default_rng(27).choice(m, size=128, replace=False), [0, m - 1]])
    Xv = WL.bf16_values(X).astype(np.float64)
    Y_ref, B = O.gemm(of, blocks, m, k, Xv, rows=rows)
    check_products(Y[:, rows], Y_ref, B, f"gemm {fmt} 64-token tiles")
    check_all_rows(Y, Xv, O.dequant(of, blocks, m, k).astype(np.float64), f"gemm {fmt} 64-token tiles")


@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: NAMES[f])
@pytest.mark.parametrize("n", [3, 24, 40, 130])
def test_gemm_single_super_block(q, fmt, n):
    # K = 256: one super-block (eight Q4_0 blocks), so every K-split and
    # pipelining path degenerates
    m, k = 70, 256
    w = mixed_blocks(m, k, 13)
    blocks = O.quantize(fmt, w)
    X = WL.bf16_bits(np.random.default_rng(14).standard_normal((n, k)).astype(np.float32))
    Y = host(q.gemm(dev(blocks), fmt, m, k, dev_bf16(X)))
    Y_ref, B = O.gemm(fmt, blocks, m, k, WL.bf16_values(X).astype(np.float64))
    check_products(Y, Y_ref, B, f"gemm {NAMES[fmt]} k=256 n={n}")


_DEQ = {}


def dequant_f64(fmt, blocks, m, k, key):
    """The oracle's rebuilt weights as float64 (cached per workload: the
    full-size prefill matrices are rebuilt once per format and shape)."""
    if key not in _DEQ:
        _DEQ.clear()
        _DEQ[key] = O.dequant(fmt, blocks, m, k).astype(np.float64)
    return _DEQ[key]


def check_all_rows(Y, Xv, Wd, what):
    """Every output of a product against numpy's float64 matmul of the
    rebuilt weights (a textbook routine on the oracle's dequantized values)
    and the bound sum |x| |w| of the same shape."""
    check_products(Y, Xv @ Wd.T, np.abs(Xv) @ np.abs(Wd).T, what + " (all rows)")


@pytest.mark.parametrize("shape", ["up", "down"])
@pytest.mark.parametrize("n", [16, 64, 512])
def test_gemm_prefill_config(q, shape, n):
    w, X = WL.sb4_prefill(shape, n)
    m, k = w.shape
    blocks = O.quantize_sb4(w)
    bd = q.quantize(dev(w), q.SB4)
    assert np.array_equal(host(bd), blocks)
    Y = host(q.gemm(bd, q.SB4, m, k, dev_bf16(X)))
    rows = np.random.default_rng(n).choice(m, size=64 if n == 512 else 256, replace=False)
    rows = np.concatenate([rows, [0, m - 1]])
    Xv = WL.bf16_values(X).astype(np.float64)
    Y_ref, B = O.gemm(O.SB4, blocks, m, k, Xv, rows=rows)
    check_products(Y[:, rows], Y_ref, B, f"gemm {shape} n={n}")
    check_all_rows(Y, Xv, dequant_f64(O.SB4, blocks, m, k, ("sb4", shape)), f"gemm {shape} n={n}")


@pytest.mark.parametrize("n", [16, 64, 512])
def test_gemm_q4_k_prefill_shape(q, n):
    w, X = WL.sb4_prefill("up", n)
    m, k = w.shape
    blocks = O.quantize_q4_k(w)
    bd = q.quantize(dev(w), q.Q4_K)
    assert np.array_equal(host(bd), blocks)
    Y = host(q.gemm(bd, q.Q4_K, m, k, dev_bf16(X)))
    rows = np.random.default_rng(n + 1).choice(m, size=64 if n == 512 else 256, replace=False)
    rows = np.concatenate([rows, [0, m - 1]])
    Xv = WL.bf16_values(X).astype(np.float64)
    Y_ref, B = O.gemm(O.Q4_K, blocks, m, k, Xv, rows=rows)
    check_products(Y[:, rows], Y_ref, B, f"gemm q4k n={n}")
    check_all_rows(Y, Xv, dequant_f64(O.Q4_K, blocks, m, k, ("q4k", "up")), f"gemm q4k n={n}")


# ------------------------------------------- group-128 W4 weights, int8 activations
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_quantize_w4g128_bit_exact(q, dtype):
    # 16 x 2304: 288 groups (18 workgroups); near-tie rows exercise the exact branch
    for w in (mixed_blocks(16, 2304, 31), near_ties(7, 2304, 32)):
        d, h = gpu_input(w, dtype)
        got = host(q.quantize(d, q.W4G128))
        assert np.array_equal(got, O.quantize_w4g128(h)), f"first mismatch at byte {np.argmax(got != O.quantize_w4g128(h))}"


@pytest.mark.parametrize("ot", ["f32", "f16", "bf16"])
def test_dequant_w4g128_bit_exact(q, ot):
    rows, k = 5, 128 * 11
    rng = np.random.default_rng(33)
    codes = rng.integers(0, 256, rows * k // 2, dtype=np.uint8)
    sc = rng.integers(0, 0x7C00, rows * k // 128).astype(np.uint16)
    sc |= (rng.integers(0, 2, sc.size) << 15).astype(np.uint16)
    for blocks in (np.concatenate([codes, sc.view(np.uint8)]), O.quantize_w4g128(mixed_blocks(rows, k, 34))):
        dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[ot]
        got = q.dequant(dev(blocks), q.W4G128, rows, k, dt)
        ref = O.dequant(O.W4G128, blocks, rows, k)
        if ot == "f32":
            assert np.array_equal(host(got).view(np.uint32), ref.view(np.uint32))
        elif ot == "f16":
            assert np.array_equal(host(got).view(np.uint16), ref.astype(np.float16).view(np.uint16))
        else:
            refb = torch.from_numpy(ref).to(torch.bfloat16).view(torch.int16).numpy()
            assert np.array_equal(host(got.view(torch.int16)), refb)


def act_rows(n, k, seed):
    """Token rows: gaussian, heavy-tailed, exact ties of the int8 grid, zeros."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, k)).astype(np.float32)
    if n > 1:
        x[1] = rng.standard_t(2, k)
    if n > 2:  # max 127 * 2^-4: every multiple of 2^-5 is a tie or a grid point
        x[2] = (rng.integers(-254, 255, k) / 2.0) * 2.0 ** -4
        x[2, 0] = 127 * 2.0 ** -4
    if n > 3:
        x[3] = 0.0
    return x


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_quantize_act_i8_bit_exact(q, dtype):
    x = act_rows(6, 2304, 35)
    d, h = gpu_input(x, dtype)
    xq, s = q.quantize_act_i8(d)
    xq_ref, s_ref = O.quantize_act_i8(h)
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(xq), xq_ref)


def w4a8_case(q, m, k, n, seed, rows=None):
    w = mixed_blocks(m, k, seed)
    blocks = O.quantize_w4g128(w)
    x = act_rows(n, k, seed + 1)
    xq_ref, s_ref = O.quantize_act_i8(x)
    xq, s = q.quantize_act_i8(dev(x))
    assert np.array_equal(host(xq), xq_ref) and np.array_equal(host(s), s_ref)
    Y = host(q.gemm_w4a8(dev(blocks), m, k, xq, s))
    Y_ref, B = O.gemm_w4a8(blocks, m, k, xq_ref, s_ref, rows=rows)
    check_products(Y if rows is None else Y[:, rows], Y_ref, B, f"w4a8 {m}x{k} n={n}")


# one token: chunks per lane 1..8 (k = 128 .. 16384) and 1..3 rows per wave
# (12-wave workgroups with 3 or 4 rows per wave beyond 32 rows per CU at
# k = 4096); k = 16512 takes the matrix-core path with n = 1
@pytest.mark.parametrize("shape", [(37, 128), (150, 2304), (300, 4096), (8704, 4096), (11008, 4096), (12300, 4096), (77, 11008),
                                   (600, 14336), (40, 16384), (20, 16512)], ids=lambda s: f"{s[0]}x{s[1]}")
def test_gemv_w4a8(q, shape):
    m, k = shape
    w4a8_case(q, m, k, 1, 36)


@pytest.mark.parametrize("n", [2, 5, 16, 24, 32, 33, 40, 64, 100, 200])
def test_gemm_w4a8(q, n):
    w4a8_case(q, 150, 2304, n, 37)


@pytest.mark.parametrize("n", [3, 20, 130])
def test_gemm_w4a8_split_k(q, n):
    w4a8_case(q, 40, 14336, n, 38)


@pytest.mark.parametrize("n", [2, 20, 40, 130])
def test_gemm_w4a8_single_group(q, n):
    # k = 128: one group, one stage
    w4a8_case(q, 70, 128, n, 40)


@pytest.mark.parametrize("n", [5, 16, 40, 300])
def test_gemm_w4a8_odd_group_count(q, n):
    # k = 9 groups: the K slices of the small-N kernel end ragged (4 + 4 + 1);
    # the wide kernel stages one group at a time
    w4a8_case(q, 200, 1152, n, 39)


@pytest.mark.parametrize("n", [16, 32, 64, 512])
def test_gemm_w4a8_prefill_shape(q, n):
    w, X = WL.sb4_prefill("up", n)
    m, k = w.shape
    blocks = O.quantize_w4g128(w)
    bd = q.quantize(dev(w), q.W4G128)
    assert np.array_equal(host(bd), blocks)
    x = WL.bf16_values(X).astype(np.float32)
    xq_ref, s_ref = O.quantize_act_i8(x)
    xq, s = q.quantize_act_i8(dev_bf16(X))
    assert np.array_equal(host(xq), xq_ref) and np.array_equal(host(s), s_ref)
    Y = host(q.gemm_w4a8(bd, m, k, xq, s))
    rows = np.random.default_rng(n + 2).choice(m, size=64 if n == 512 else 256, replace=False)
    rows = np.concatenate([rows, [0, m - 1]])
    Y_ref, B = O.gemm_w4a8(blocks, m, k, xq_ref, s_ref, rows=rows)
    check_products(Y[:, rows], Y_ref, B, f"w4a8 prefill n={n}")
    # every row: the rebuilt int8 activations (code times the token's scale, R31)
    Xv = xq_ref.astype(np.float64) * s_ref.astype(np.float64)[:, None]
    check_all_rows(Y, Xv, dequant_f64(O.W4G128, blocks, m, k, ("w4g128", "up")), f"w4a8 prefill n={n}")


def test_w4a8_token_slices(q):
    # slices of the int8 tokens and of their fp32 scales (4-byte aligned) are
    # valid inputs and give those tokens' rows of the product
    m, k, n = 96, 1024, 9
    w = mixed_blocks(m, k, 41)
    blocks = O.quantize_w4g128(w)
    bd = dev(blocks)
    x = act_rows(n, k, 42)
    xq, s = q.quantize_act_i8(dev(x))
    xq_ref, s_ref = O.quantize_act_i8(x)
    Y_ref, B = O.gemm_w4a8(blocks, m, k, xq_ref, s_ref)
    for a, b in ((1, 2), (3, 9), (5, 6)):
        Ys = host(q.gemm_w4a8(bd, m, k, xq[a:b], s[a:b]))
        check_products(Ys, Y_ref[a:b], B[a:b], f"w4a8 tokens {a}:{b}")


# ------------------------------------------------------- streams and graphs
@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: NAMES[f])
@pytest.mark.parametrize("m,k,n", [(150, 2304, 16), (40, 14336, 20), (40, 14336, 130), (150, 2304, 100)])
def test_gemm_deterministic(q, fmt, m, k, n):
    # reproducible products: shapes whose K is split over the grid by default
    # (one stage per workgroup, the streaming and the wide kernels) give
    # bitwise equal outputs over repeated calls, within the bound
    w = mixed_blocks(m, k, 41)
    blocks = O.quantize(fmt, w)
    X = WL.bf16_bits(np.random.default_rng(42).standard_normal((n, k)).astype(np.float32))
    bd, Xd = dev(blocks), dev_bf16(X)
    try:
        q.set_deterministic(True)
        runs = [host(q.gemm(bd, fmt, m, k, Xd)) for _ in range(4)]
    finally:
        q.set_deterministic(False)
    for Y in runs[1:]:
        assert np.array_equal(Y.view(np.uint32), runs[0].view(np.uint32))
    Y_ref, B = O.gemm(fmt, blocks, m, k, WL.bf16_values(X).astype(np.float64))
    check_products(runs[0], Y_ref, B, f"deterministic gemm {NAMES[fmt]} n={n}")


@pytest.mark.parametrize("m,k,n", [(150, 2304, 16), (40, 14336, 40), (40, 14336, 130)])
def test_gemm_w4a8_deterministic(q, m, k, n):
    w = mixed_blocks(m, k, 43)
    blocks = O.quantize_w4g128(w)
    x = np.random.default_rng(44).standard_normal((n, k)).astype(np.float32)
    xq, s = O.quantize_act_i8(x)
    bd, xqd, sd = dev(blocks), dev(xq), dev(s)
    try:
        q.set_deterministic(True)
        runs = [host(q.gemm_w4a8(bd, m, k, xqd, sd)) for _ in range(4)]
    finally:
        q.set_deterministic(False)
    for Y in runs[1:]:
        assert np.array_equal(Y.view(np.uint32), runs[0].view(np.uint32))
    Y_ref, B = O.gemm_w4a8(blocks, m, k, xq, s)
    check_products(runs[0], Y_ref, B, f"deterministic gemm_w4a8 n={n}")


def test_threads_on_their_own_streams(q):
    # the C ABI keeps no per-call state: four host threads, each calling every
    # product on a stream of its own at the same time (ctypes releases the
    # interpreter lock during each call), get the bytes and products that the
    # calls give one at a time
    import threading
    m, k = 300, 4096
    w = mixed_blocks(m, k, 55)
    wd = dev(w)
    xs = [dev(np.random.default_rng(56 + t).standard_normal(k).astype(np.float16)) for t in range(4)]
    Xs = [dev_bf16(WL.bf16_bits(np.random.default_rng(60 + t).standard_normal((24, k)).astype(np.float32)))
          for t in range(4)]
    # expected results, one call at a time
    b_ref = q.quantize(wd, q.SB4)
    want = [(host(q.gemv(b_ref, q.SB4, m, k, xs[t])), host(q.gemm(b_ref, q.SB4, m, k, Xs[t]))) for t in range(4)]
    b_ref = host(b_ref)
    got, errors = [None] * 4, []

    def work(t):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                out = []
                for _ in range(10):
                    b = q.quantize(wd, q.SB4, stream=st)
                    y = q.gemv(b, q.SB4, m, k, xs[t], stream=st)
                    (yb,) = q.gemv_batch(q.SB4, k, [(b, m, xs[t])], stream=st)
                    Y = q.gemm(b, q.SB4, m, k, Xs[t], stream=st)
                    out.append((b, y, yb, Y))
            st.synchronize()
            got[t] = [(host(b), host(y), host(yb), host(Y)) for b, y, yb, Y in out]
        except Exception as e:  # reported below, in the test's own thread
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(120)
    assert not errors, errors
    for t in range(4):
        y_want, Y_want = want[t]
        for b, y, yb, Y in got[t]:
            assert np.array_equal(b, b_ref)
            assert np.array_equal(y.view(np.uint32), y_want.view(np.uint32))
            assert np.allclose(yb, y_want, rtol=0, atol=1e-4 * float(np.max(np.abs(y_want))))
            assert np.allclose(Y, Y_want, rtol=0, atol=1e-4 * float(np.max(np.abs(Y_want))))


def test_side_stream(q):
    # every step enqueues on the stream it is handed: the same calls on a
    # second stream give the oracle's bytes and products
    m, k = 150, 2304
    w = mixed_blocks(m, k, 51)
    x = np.random.default_rng(52).standard_normal(k).astype(np.float16)
    X = WL.bf16_bits(np.random.default_rng(53).standard_normal((20, k)).astype(np.float32))
    xa = act_rows(5, k, 54)
    wd, xd, Xd, xad = dev(w), dev(x), dev_bf16(X), dev(xa)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):  # (the binding's default is the current stream)
        b = q.quantize(wd, q.SB4, stream=side)
        bw = q.quantize(wd, q.W4G128, stream=side)
        deq = q.dequant(b, q.SB4, m, k, stream=side)
        y = q.gemv(b, q.SB4, m, k, xd, stream=side)
        Y = q.gemm(b, q.SB4, m, k, Xd, stream=side)
        xq, s = q.quantize_act_i8(xad, stream=side)
        Yw = q.gemm_w4a8(bw, m, k, xq, s, stream=side)
    side.synchronize()
    b_ref = O.quantize_sb4(w)
    assert np.array_equal(host(b), b_ref)
    assert np.array_equal(host(bw), O.quantize_w4g128(w))
    assert np.array_equal(host(deq).view(np.uint32), O.dequant(O.SB4, b_ref, m, k).view(np.uint32))
    y_ref, yb = O.gemv(O.SB4, b_ref, m, k, x.astype(np.float64))
    check_products(host(y), y_ref, yb, "side-stream gemv")
    Y_ref, Yb = O.gemm(O.SB4, b_ref, m, k, WL.bf16_values(X).astype(np.float64))
    check_products(host(Y), Y_ref, Yb, "side-stream gemm")
    xq_ref, s_ref = O.quantize_act_i8(xa)
    Yw_ref, Ywb = O.gemm_w4a8(O.quantize_w4g128(w), m, k, xq_ref, s_ref)
    check_products(host(Yw), Yw_ref, Ywb, "side-stream w4a8")


def test_graph_replay(q):
    # the products captured once into a HIP graph and replayed: the split-K
    # GEMMs clear Y with a fill kernel inside the graph before adding their
    # partial sums, so every replay must reproduce the product from a Y that
    # eager work in between has overwritten
    m, k = 150, 2304
    w = mixed_blocks(m, k, 55)
    b_ref, bw_ref = O.quantize_sb4(w), O.quantize_w4g128(w)
    x = np.random.default_rng(56).standard_normal(k).astype(np.float16)
    X = WL.bf16_bits(np.random.default_rng(57).standard_normal((16, k)).astype(np.float32))
    X64 = WL.bf16_bits(np.random.default_rng(58).standard_normal((40, k)).astype(np.float32))
    xa = act_rows(5, k, 59)
    b, bw, xd, Xd, X64d = dev(b_ref), dev(bw_ref), dev(x), dev_bf16(X), dev_bf16(X64)
    xq, s = q.quantize_act_i8(dev(xa))
    y = torch.empty(m, device="cuda")
    Y = torch.empty((16, m), device="cuda")
    Y64 = torch.empty((40, m), device="cuda")
    Yw = torch.empty((5, m), device="cuda")
    cap = torch.cuda.Stream()

    def step():
        q.gemv(b, q.SB4, m, k, xd, out=y)
        q.gemm(b, q.SB4, m, k, Xd, out=Y)        # one stage per workgroup, K split 5 ways
        q.gemm(b, q.SB4, m, k, X64d, out=Y64)    # streaming kernel
        q.gemm_w4a8(bw, m, k, xq, s, out=Yw)     # K split 5 ways

    torch.cuda.synchronize()
    with torch.cuda.stream(cap):
        step()  # warm-up on the capture stream
    cap.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        step()
    y_ref, yb = O.gemv(O.SB4, b_ref, m, k, x.astype(np.float64))
    Y_ref, Yb = O.gemm(O.SB4, b_ref, m, k, WL.bf16_values(X).astype(np.float64))
    Y64_ref, Y64b = O.gemm(O.SB4, b_ref, m, k, WL.bf16_values(X64).astype(np.float64))
    xq_ref, s_ref = O.quantize_act_i8(xa)
    Yw_ref, Ywb = O.gemm_w4a8(bw_ref, m, k, xq_ref, s_ref)
    for rep in range(3):
        for t in (y, Y, Y64, Yw):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check_products(host(y), y_ref, yb, f"graph gemv, replay {rep}")
        check_products(host(Y), Y_ref, Yb, f"graph gemm n=16, replay {rep}")
        check_products(host(Y64), Y64_ref, Y64b, f"graph gemm n=40, replay {rep}")
        check_products(host(Yw), Yw_ref, Ywb, f"graph w4a8 n=5, replay {rep}")
