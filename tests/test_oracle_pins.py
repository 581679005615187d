"""Pins of the CPU oracle to what the pages and the mathematics fix.

Every test here checks the oracle against something other than itself: values
the pages print (tests/golden/), closed forms, library routines (numpy's and
torch's IEEE conversions, Python's decimal rounding, numpy's float64 matmul)
or brute force over every admissible code.  No GPU is involved.

Pages:
  K-quants blog   "GGUF K-quants" (hugo-blog-2v1.pages.dev/2025/gguf-k-quants/)
  Q4_0 chapter    "GGUF 量化内幕 第4章 Q4_0：块量化的起点" (sxkj888.cn)
  TurboQuant article  the W4A8 page (codechina.net), sections 2.1 and 2.2

The Q4_K form (chapter section 4.6) has no worked example on the pages: its
pins are a hand-derived block (tests/golden/q4_k_block.txt), brute force over
every 6-bit and 4-bit code, the error bound its rebuilt range implies, the
degenerate blocks and numpy's matmul for the products.  The group-128 W4A8
scheme (TurboQuant article) is pinned the same way, and its product against
an exact integer-and-rational evaluation.
"""
import decimal
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import workloads as WL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition("=")
            nums = [float(t) for t in rest.split()]
            vals[key.strip()] = nums if len(nums) > 1 else nums[0]
    return vals


def f16(v):
    """numpy's IEEE binary16 conversion (round to nearest even) of a float32."""
    return int(np.array([v], dtype=np.float32).astype(np.float16).view(np.uint16)[0])


def f16val(bits):
    return float(np.array([bits], dtype=np.uint16).view(np.float16).astype(np.float32)[0])


def f32(v):
    return np.float32(v)


def nibbles(qs16):
    """codes of the 32 weights of one 16-byte group, in weight order."""
    qs = np.asarray(qs16, dtype=np.uint8)
    return np.concatenate([qs & 0x0F, qs >> 4]).astype(np.int64)


# --------------------------------------------------------------------------
# sizes and storage arithmetic (closed forms printed on the pages)
# --------------------------------------------------------------------------
def test_block_sizes_and_bits_per_weight():
    # Q4_0 chapter 4.1.2: 2 + 16 = 18 bytes for 32 weights, 4.5 bit/weight
    assert O.block_elems(O.Q4_0) == 32 and O.block_bytes(O.Q4_0) == 18
    assert O.block_bytes(O.Q4_0) * 8 / 32 == 4.5
    # Q4_0 chapter intro: 18 of 128 bytes, "about 14%" of fp32
    assert round(100 * 18 / 128) == 14
    # K-quants blog storage table: 4 + 80/256 = 4.3125 bit/weight
    assert O.block_elems(O.SB4) == 256 and O.block_bytes(O.SB4) == 138
    assert O.block_bytes(O.SB4) * 8 / 256 == 4.3125
    # Type 1 adds 8 INT8 offsets + one fp16 super-offset: 4 + 160/256
    assert O.block_elems(O.SB4_AFFINE) == 256 and O.block_bytes(O.SB4_AFFINE) == 148
    assert O.block_bytes(O.SB4_AFFINE) * 8 / 256 == 4.625


def test_constant_overhead_arithmetic():
    # K-quants blog storage table: eight fp16 scales = 128 bit before, eight
    # INT8 + one fp16 = 80 bit after, 48 bit saved per super-block.
    const_bits_sb = (O.block_bytes(O.SB4) - 256 // 2) * 8
    assert 8 * 16 == 128 and const_bits_sb == 80 and 128 - const_bits_sb == 48
    # 16e9 parameters: 5e8 blocks of 32; 6 bit saved per block-constant
    # (16 -> 80/8 = 10) is 3e9 bit = 375 MB; Type 1 saves the same on alpha.
    blocks = 16e9 / 32
    assert blocks == 5e8
    saved_per_const = 16 - const_bits_sb / 8
    assert saved_per_const == 6
    assert blocks * saved_per_const / 8 == 375e6
    # legacy Type 1 (fp16 scale + fp16 offset per 32) = 2 GB of constants;
    # Type 1 super-blocks need 20 constant bytes per 256 weights = 1.25 GB,
    # which the page rounds to "about 1 GB" (2 GB - 2 x 375 MB).
    legacy = blocks * 4
    t1 = 16e9 / 256 * (O.block_bytes(O.SB4_AFFINE) - 128)
    assert legacy == 2e9 and t1 == 1.25e9 and legacy - 2 * 375e6 == t1


# --------------------------------------------------------------------------
# number formats, against library routines
# --------------------------------------------------------------------------
def test_f16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([O.f16_to_f32(b) for b in bits], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f16_encode_vs_numpy():
    fin = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)
    vals = fin.view(np.float16).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2  # every tie between neighbours (exact in f32)
    mids32 = mids.astype(np.float32)
    up = np.nextafter(mids32, np.float32(np.inf))
    dn = np.nextafter(mids32, np.float32(0))
    rng = np.random.default_rng(7)
    rnd = (np.exp(rng.uniform(np.log(1e-9), np.log(7e4), 20000))).astype(np.float32)
    cand = np.concatenate([vals.astype(np.float32), mids32, up, dn, rnd,
                           np.float32([65504, 65519.996, 65520, 1e6, 0.0])])
    cand = np.concatenate([cand, -cand])
    with np.errstate(over="ignore"):
        ref = cand.astype(np.float16).view(np.uint16)
    got = np.array([O.f32_to_f16(v) for v in cand], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_codec_vs_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    v = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (np.exp(rng.uniform(-80, 80, 5000))).astype(np.float32),
        np.float32([1e-40, 3e-39, 1.0, 3.4e38, 0.0]),
    ])
    # ties: values exactly halfway between two bf16 neighbours
    b = rng.integers(0x0080, 0x7F00, 5000).astype(np.uint32)
    ties = ((b << 16) | 0x8000).astype(np.uint32).view(np.float32)
    v = np.concatenate([v, ties, -v, -ties])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([O.f32_to_bf16(x) for x in v], dtype=np.uint16)
    assert np.array_equal(got, ref)
    back = np.array([O.bf16_to_f32(x) for x in ref], dtype=np.float32)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_round_half_away_vs_decimal():
    rng = np.random.default_rng(3)
    vals = list(np.float32([0.5, 1.5, 2.5, -0.5, -2.5, 0.49999997, -0.49999997, 7.5, -8.5,
                            126.5, -126.5, 8388607.5, 0.0, -0.0]))
    vals += list((rng.standard_normal(5000) * 50).astype(np.float32))
    vals += list((rng.integers(-300, 300, 2000) + 0.5).astype(np.float32))
    for v in vals:
        ref = float(decimal.Decimal(float(v)).quantize(decimal.Decimal(1), rounding=decimal.ROUND_HALF_UP))
        assert O.rha(v) == ref, v


# --------------------------------------------------------------------------
# byte layout, from hand-made blocks
# --------------------------------------------------------------------------
def test_q4_0_nibble_order_and_minus_8():
    # Q4_0 chapter 4.2.1/4.2.2/4.3: byte j holds weight j (low nibble) and
    # weight j+16 (high nibble); value = d * (code - 8).
    blk = np.zeros(18, dtype=np.uint8)
    blk[0:2] = np.array([0x3C00], dtype="<u2").view(np.uint8)  # d = 1.0
    for j in range(16):
        blk[2 + j] = j | ((15 - j) << 4)
    y = O.dequant(O.Q4_0, blk, 1, 32)[0]
    assert list(y[:16]) == [j - 8 for j in range(16)]
    assert list(y[16:]) == [7 - j for j in range(16)]
    # a scale of -1.25 (fp16 0xBD00) flips the signs
    blk[0:2] = np.array([0xBD00], dtype="<u2").view(np.uint8)
    y = O.dequant(O.Q4_0, blk, 1, 32)[0]
    assert y[0] == 10.0 and y[8] == 0.0 and y[16] == -8.75


def test_sb4_type0_layout():
    # reading R8/R9: [S16][sc x8 int8][qs of sub-block 0..7, 16 bytes each]
    blk = np.zeros(138, dtype=np.uint8)
    blk[0:2] = np.array([0x3800], dtype="<u2").view(np.uint8)  # S = 0.5
    sc = np.array([1, 2, -3, 4, 127, -127, 0, 9], dtype=np.int8)
    blk[2:10] = sc.view(np.uint8)
    rng = np.random.default_rng(5)
    qs = rng.integers(0, 256, 128, dtype=np.uint8)
    blk[10:] = qs
    y = O.dequant(O.SB4, blk, 1, 256)[0]
    for j in range(8):
        n = nibbles(qs[16 * j:16 * j + 16])
        assert np.array_equal(y[32 * j:32 * j + 32], 0.5 * sc[j] * (n - 8))


def test_sb4_type1_layout():
    # reading R8/R10/R14: [Ss16][Sa16][sc x8][ac x8][qs x128], w = Ss*sc*n + Sa*ac
    blk = np.zeros(148, dtype=np.uint8)
    blk[0:4] = np.array([0x3400, 0x3C00], dtype="<u2").view(np.uint8)  # 0.25, 1.0
    sc = np.array([4, 8, 1, 0, 127, 3, 2, 5], dtype=np.int8)
    ac = np.array([-1, 0, 2, -127, 5, 7, -3, 1], dtype=np.int8)
    blk[4:12] = sc.view(np.uint8)
    blk[12:20] = ac.view(np.uint8)
    rng = np.random.default_rng(6)
    qs = rng.integers(0, 256, 128, dtype=np.uint8)
    blk[20:] = qs
    y = O.dequant(O.SB4_AFFINE, blk, 1, 256)[0]
    for j in range(8):
        n = nibbles(qs[16 * j:16 * j + 16])
        assert np.array_equal(y[32 * j:32 * j + 32], 0.25 * sc[j] * n + ac[j])


# --------------------------------------------------------------------------
# the pages' worked examples
# --------------------------------------------------------------------------
def test_kquants_worked_example():
    g = read_golden("kquants_worked_example.txt")
    s16 = [f16(v) for v in g["scales"]]  # "each block's scale is an FP16 value"
    s = np.array([f16val(b) for b in s16], dtype=np.float32)
    codes, S16, Su = O.meta_int8(s)
    # reading R2: against the stored super-scale every printed code comes out
    assert list(codes) == [int(c) for c in g["codes"]]
    assert S16 == 0x15CF and round(Su, 5) == g["s_meta_printed"]
    err = np.abs(codes.astype(np.float64) * Su - s)
    assert err.max() <= g["error_max"]
    # with the page's printed (rounded) super-scale the quotient column and the
    # rebuilt/error columns match the tables to their printed precision;
    # 0.11/0.00142 = 77.46 is printed 77.5 and then rounded to 78 on the page,
    # while a single rounding gives 77 (the page rounds twice).
    c2, _, Su2 = O.meta_int8(s, S_forced=g["s_meta_printed"])
    # the printed quotients are the decimal scales over 0.00142, to one decimal
    dec = np.array(g["scales"]) / g["s_meta_printed"]
    assert np.allclose(np.round(dec, 1), g["quotients_printed"])
    # the fp16 scales move them by less than 0.06
    q = s / np.float32(Su2)
    assert np.all(np.abs(q - np.array(g["quotients_printed"])) <= 0.06)
    expect = [int(c) for c in g["codes"]]
    expect[2] = 77
    assert list(c2) == expect
    rebuilt = np.array(g["codes"]) * g["s_meta_printed"]
    assert np.allclose(np.round(rebuilt, 4), g["rebuilt_printed"])
    assert np.allclose(np.round(np.abs(rebuilt - np.array(g["scales"])), 4), g["errors_printed"])
    assert g["error_min"] <= np.round(np.abs(rebuilt - np.array(g["scales"])), 4).min()


def test_kquants_worked_example_through_a_super_block():
    # 256 weights whose eight sub-block scales are the page's eight FP16
    # scales: sub-block j holds 7*s_j once (its absmax) and small values.
    g = read_golden("kquants_worked_example.txt")
    w = np.zeros((1, 256), dtype=np.float32)
    rng = np.random.default_rng(9)
    for j, v in enumerate(g["scales"]):
        sj = f16val(f16(v))
        w[0, 32 * j:32 * j + 32] = rng.uniform(-6, 6, 32).astype(np.float32) * np.float32(sj)
        w[0, 32 * j + 5] = np.float32(7.0 * sj)  # exact: 11-bit value times 7
    blk = O.quantize_sb4(w)
    assert int(blk[0:2].view("<u2")[0]) == 0x15CF
    assert list(blk[2:10].view(np.int8)) == [int(c) for c in g["codes"]]


def test_q4_0_outlier_example():
    g = read_golden("q4_0_outlier_demo.txt")
    n = int(g["small_count"])
    vals = [g["small_scale"] * (i - 15) / 15 for i in range(n)] + [g["outlier"]]
    w = np.array(vals, dtype=np.float32).reshape(1, 32)
    # the chapter's own quantizer (section 4.4): d = 10 / -8
    ref = O.quantize_q4_0_ref(w)
    assert f16val(int(ref[0:2].view("<u2")[0])) == g["ref_scale"]
    codes = nibbles(ref[2:18])
    assert set(codes[:31]) == {int(g["ref_small_code"])}
    assert codes[31] == int(g["ref_outlier_code"])
    # the absmax/7 rule (reading R1): the same collapse, the outlier on code 15
    b = O.quantize_q4_0(w)
    codes = nibbles(b[2:18])
    assert set(codes[:31]) == {8} and codes[31] == 15
    y = O.dequant(O.Q4_0, b, 1, 32)[0]
    assert np.all(y[:31] == 0) and abs(y[31] - 10.0) < 10.0 / 7 / 2


def read_golden_raw(name):
    """key = value lines as strings (for fixtures holding dicts and hex bytes)."""
    vals = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                key, _, rest = line.partition("=")
                vals[key.strip()] = rest.strip()
    return vals


def _listing_block(values):
    w = np.zeros((1, 32), dtype=np.float32)
    for i, v in values.items():
        w[0, int(i)] = v
    return w


def test_q4_0_listing_cap_first_extreme_and_reciprocal():
    # "GGUF 量化内幕 第4章 Q4_0" 4.4: hand-derived bytes for the parts of the
    # listing no printed example reaches (tests/golden/q4_0_listing_cap_and_ties.txt)
    import ast
    g = read_golden_raw("q4_0_listing_cap_and_ties.txt")
    for name in ("cap", "first"):
        got = O.quantize_q4_0_ref(_listing_block(ast.literal_eval(g[f"{name}_values"])))
        want = bytes.fromhex(g[f"{name}_bytes"].replace(" ", ""))
        assert got.tobytes() == want, f"block {name}: {got.tobytes().hex()} != {want.hex()}"
    E = np.array([int(g["recip_e_bits"], 16)], np.uint32).view(np.float32)[0]
    X = np.array([int(g["recip_x_bits"], 16)], np.uint32).view(np.float32)[0]
    got = O.quantize_q4_0_ref(_listing_block({0: E, 7: X}))
    codes = nibbles(got[2:18])
    assert codes[0] == 0 and codes[7] == int(g["recip_code_x"])
    assert codes[7] != int(g["recip_code_if_divided"])


# --------------------------------------------------------------------------
# brute force: every stored code is the best admissible one
# --------------------------------------------------------------------------
def best_code(t, lo, hi):
    """argmin over integers c in [lo, hi] of |t - c|, ties away from zero."""
    t = Fraction(float(t))
    best = None
    for c in range(lo, hi + 1):
        key = (abs(t - c), -abs(c))
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def tiny_blocks(rng, nblk, size):
    """blocks of several flavours: gaussian, heavy tails, exact ties, subnormal scales."""
    out = []
    for i in range(nblk):
        kind = i % 5
        if kind == 0:
            b = rng.standard_normal(size) * 0.02
        elif kind == 1:
            b = rng.standard_t(2, size) * 0.05
        elif kind == 2:  # values on exact half steps of a power-of-two scale
            b = (rng.integers(-15, 16, size) / 2.0) * 2.0 ** -6
            b[0] = 7 * 2.0 ** -6
        elif kind == 3:
            b = rng.standard_normal(size) * 1e-6  # fp16-subnormal scales
        else:
            b = rng.uniform(-3, 3, size)
            b[rng.integers(0, size, 3)] = 0.0
        out.append(b.astype(np.float32))
    return np.stack(out)


def test_brute_force_q4_0_codes():
    rng = np.random.default_rng(21)
    w = tiny_blocks(rng, 60, 32)
    blocks = O.quantize_q4_0(w).reshape(-1, 18)
    for b in range(w.shape[0]):
        d16 = int(blocks[b, 0:2].view("<u2")[0])
        amax = np.float32(np.max(np.abs(w[b])))
        assert d16 == f16(amax / np.float32(7.0))
        d = np.float32(f16val(d16))
        codes = nibbles(blocks[b, 2:])
        for i in range(32):
            t = np.float32(0.0) if d == 0 else w[b, i] / d  # IEEE fp32 quotient
            assert codes[i] - 8 == best_code(t, -8, 7), (b, i)


def test_brute_force_meta_int8():
    rng = np.random.default_rng(22)
    for trial in range(300):
        mag = 10.0 ** rng.uniform(-7, 2)
        s16 = [f16(np.float32(v)) for v in np.abs(rng.standard_normal(8)) * mag]
        s = np.array([f16val(b) for b in s16], dtype=np.float32)
        codes, S16, Su = O.meta_int8(s)
        assert S16 == f16(np.float32(s.max()) / np.float32(127.0))
        for i in range(8):
            t = np.float32(0.0) if Su == 0 else s[i] / np.float32(Su)
            assert codes[i] == best_code(t, -127, 127)


def test_brute_force_type1_codes():
    rng = np.random.default_rng(23)
    w = tiny_blocks(rng, 10, 256)
    blk = O.quantize_sb4(w, affine=True).reshape(-1, 148)
    for b in range(w.shape[0]):
        s = np.zeros(8, np.float32)
        a = np.zeros(8, np.float32)
        for j in range(8):
            x = w[b, 32 * j:32 * j + 32]
            s[j] = f16val(f16((x.max() - x.min()) / np.float32(15.0)))
            a[j] = f16val(f16(x.min()))
            codes = nibbles(blk[b, 20 + 16 * j:36 + 16 * j])
            for i in range(32):
                t = np.float32(0.0) if s[j] == 0 else (x[i] - a[j]) / s[j]
                assert codes[i] == best_code(t, 0, 15), (b, j, i)
        Ss, Sa = (f16val(int(v)) for v in blk[b, 0:4].view("<u2"))
        assert int(blk[b, 0:2].view("<u2")[0]) == f16(s.max() / np.float32(127))
        assert int(blk[b, 2:4].view("<u2")[0]) == f16(np.abs(a).max() / np.float32(127))
        sc = blk[b, 4:12].view(np.int8)
        ac = blk[b, 12:20].view(np.int8)
        for j in range(8):
            ts = np.float32(0) if Ss == 0 else s[j] / np.float32(Ss)
            ta = np.float32(0) if Sa == 0 else a[j] / np.float32(Sa)
            assert sc[j] == best_code(ts, -127, 127)
            assert ac[j] == best_code(ta, -127, 127)


# --------------------------------------------------------------------------
# properties: idempotence, agreement between formats, error bounds
# --------------------------------------------------------------------------
def test_q4_0_idempotent_when_scale_is_normal():
    w, _ = WL.q4_0_small()
    w = w[:32]
    b = O.quantize_q4_0(w)
    b2 = O.quantize_q4_0(O.dequant(O.Q4_0, b, 32, 4096))
    d16 = b.reshape(-1, 18)[:, 0:2].copy().view("<u2")[:, 0]
    normal = (d16 & 0x7C00) != 0
    assert normal.mean() > 0.99
    assert np.array_equal(b.reshape(-1, 18)[normal], b2.reshape(-1, 18)[normal])


def test_sb4_qs_idempotent():
    w, _ = WL.sb4_decode("up")
    w = w[:64]
    b = O.quantize_sb4(w).reshape(-1, 138)
    b2 = O.quantize_sb4(O.dequant(O.SB4, b.reshape(-1), 64, 4096)).reshape(-1, 138)
    sc = b[:, 2:10].view(np.int8)
    for j in range(8):
        live = sc[:, j] != 0
        assert np.array_equal(b[live, 10 + 16 * j:26 + 16 * j], b2[live, 10 + 16 * j:26 + 16 * j])


def test_super_block_codes_equal_q4_0_codes():
    w, _ = WL.sb4_decode("down")
    w = w[:16]
    sb = O.quantize_sb4(w).reshape(-1, 138)
    q4 = O.quantize_q4_0(w).reshape(-1, 8, 18)
    assert np.array_equal(sb[:, 10:].reshape(-1, 8, 16), q4[:, :, 2:])
    d = q4[:, :, 0:2].copy().view("<u2")[..., 0].astype(np.uint16).view(np.float16).astype(np.float64)
    S = sb[:, 0:2].copy().view("<u2")[:, 0].view(np.float16).astype(np.float64)
    sc = sb[:, 2:10].view(np.int8).astype(np.float64)
    assert np.all(np.abs(sc * S[:, None] - d) <= S[:, None] / 2 * (1 + 1e-6))


def test_error_bounds():
    rng = np.random.default_rng(31)
    w = (rng.standard_normal((8, 1024)) * np.exp(rng.uniform(-6, 0, (8, 1)))).astype(np.float32)
    eps = 2.0 ** -22
    # Q4_0: half a step for every weight (the clamp never bites with a normal scale)
    b = O.quantize_q4_0(w)
    y = O.dequant(O.Q4_0, b, 8, 1024)
    d = b.reshape(8, -1, 18)[:, :, 0:2].copy().view("<u2")[..., 0].view(np.float16).astype(np.float64)
    dd = np.repeat(d, 32, axis=1)
    assert np.all(np.abs(w - y) <= dd / 2 * (1 + eps) + 1e-30)
    # Type 0: first-level step/2 plus the INT8 rebuild error of the scale
    b = O.quantize_sb4(w).reshape(8, -1, 138)
    y = O.dequant(O.SB4, b.reshape(-1), 8, 1024)
    q4 = O.quantize_q4_0(w).reshape(8, -1, 18)
    d = q4[:, :, 0:2].copy().view("<u2")[..., 0].view(np.float16).astype(np.float64)
    S = b[:, :, 0:2].copy().view("<u2")[..., 0].view(np.float16).astype(np.float64)
    q = np.abs(y / np.maximum(np.repeat(b[:, :, 2:10].view(np.int8).reshape(8, -1), 32, 1) *
                              np.repeat(S, 256, 1), 1e-30))
    bound = np.repeat(d, 32, 1) / 2 + 8 * np.repeat(S, 256, 1) / 2
    assert np.all(np.abs(w - y) <= bound * (1 + 1e-5))
    assert np.all(q <= 8 + 1e-3)
    # Type 1: step/2 + 15 * Ss/2 + Sa/2 + the fp16 rounding of the offset
    b = O.quantize_sb4(w, affine=True).reshape(8, -1, 148)
    y = O.dequant(O.SB4_AFFINE, b.reshape(-1), 8, 1024)
    wb = w.reshape(8, -1, 8, 32).astype(np.float64)
    s = ((wb.max(-1) - wb.min(-1)) / 15)
    Ss = b[:, :, 0:2].copy().view("<u2")[..., 0].view(np.float16).astype(np.float64)
    Sa = b[:, :, 2:4].copy().view("<u2")[..., 0].view(np.float16).astype(np.float64)
    amin = np.abs(wb.min(-1))
    bound = (s * (1 + 2 ** -10)) / 2 + 15 * Ss[..., None] / 2 + Sa[..., None] / 2 + amin * 2 ** -11
    err = np.abs(w.reshape(8, -1, 8, 32) - y.reshape(8, -1, 8, 32)).max(-1)
    assert np.all(err <= bound * (1 + 1e-5) + 1e-30)


def test_degenerate_blocks():
    w = np.zeros((2, 256), dtype=np.float32)
    w[1, :] = np.float32(0.375)  # constant block
    q = O.quantize_q4_0(w).reshape(-1, 18)
    assert np.all(q[:8, 0:2] == 0) and np.all(q[:8, 2:] == 0x88)
    t1 = O.quantize_sb4(w, affine=True).reshape(-1, 148)
    assert np.all(t1[1, 4:12] == 0)  # zero scales
    assert np.all(t1[1, 20:] == 0)  # codes 0
    y = O.dequant(O.SB4_AFFINE, t1.reshape(-1), 2, 256)
    assert np.all(y[0] == 0)
    Sa = f16val(int(t1[1, 2:4].view("<u2")[0]))
    assert np.allclose(y[1], 0.375, atol=Sa / 2)
    t0 = O.quantize_sb4(w).reshape(-1, 138)
    assert np.all(O.dequant(O.SB4, t0.reshape(-1), 2, 256)[0] == 0)


# --------------------------------------------------------------------------
# the Q4_K form (Q4_0 chapter 4.6): y = d*s_j*q - dmin*m_j
# --------------------------------------------------------------------------
def q4k_fields(hdr12):
    """the sixteen 6-bit fields (s_0..s_7, m_0..m_7) of bytes 4..15, field i
    at bits 6i..6i+5 of the little-endian integer (reading R23)."""
    v = int.from_bytes(bytes(np.asarray(hdr12, dtype=np.uint8)), "little")
    return [(v >> (6 * i)) & 63 for i in range(16)]


def test_q4_k_hand_derived_block():
    g = read_golden("q4_k_block.txt")
    w = np.zeros((1, 256), np.float32)
    q = np.arange(32) % 16
    w[0, 0:32] = q * np.float32(63 / 256)
    w[0, 32:64] = np.float32(-63 / 32) + q * np.float32(0.125)
    assert O.block_bytes(O.Q4_K) == 144 and O.block_elems(O.Q4_K) == 256
    blk = O.quantize_q4_k(w)
    assert list(blk[0:16]) == [int(v) for v in g["header"]]
    assert list(blk[16:32]) == [int(v) for v in g["codes_sub_block_0"]]
    assert list(blk[32:48]) == [int(v) for v in g["codes_sub_block_1"]]
    assert np.all(blk[48:] == 0)
    y = O.dequant(O.Q4_K, blk, 1, 256)[0]
    assert np.array_equal(y, w[0])  # every input is on the grid
    # a hand-built block: d = 1/64, dmin = 1/2, fields from the golden file
    fields = [int(v) for v in g["block2_fields"]]
    packed = sum(v << (6 * i) for i, v in enumerate(fields)).to_bytes(12, "little")
    b2 = np.zeros(144, np.uint8)
    b2[0:4] = np.array([0x2400, 0x3800], dtype="<u2").view(np.uint8)
    b2[4:16] = np.frombuffer(packed, dtype=np.uint8)
    b2[16] = 0xF0  # sub-block 0: weight 0 code 0, weight 16 code 15
    b2[16 + 32] = 0x08  # sub-block 2, weight 0 code 8
    b2[16 + 96:16 + 112] = 0x88  # sub-block 6: all codes 8
    y2 = O.dequant(O.Q4_K, b2, 1, 256)[0]
    for i, v in zip((0, 16, 64, 65, 192, 223), g["block2_values"]):
        assert y2[i] == np.float32(v), (i, y2[i], v)


def test_brute_force_q4_k_codes():
    rng = np.random.default_rng(24)
    w = tiny_blocks(rng, 15, 256)
    blk = O.quantize_q4_k(w).reshape(-1, 144)
    for b in range(w.shape[0]):
        x = w[b].reshape(8, 32)
        lo = np.minimum(x.min(1), np.float32(0))  # reading R24
        sc = ((x.max(1) - lo) / np.float32(15)).astype(np.float32)
        mn = (-lo).astype(np.float32)
        d16, m16 = (int(v) for v in blk[b, 0:4].view("<u2"))
        assert d16 == f16(sc.max() / np.float32(63)) and m16 == f16(mn.max() / np.float32(63))
        D, Dm = np.float32(f16val(d16)), np.float32(f16val(m16))
        F = q4k_fields(blk[b, 4:16])
        for j in range(8):
            assert F[j] == best_code(np.float32(0) if D == 0 else sc[j] / D, 0, 63), (b, j)
            assert F[8 + j] == best_code(np.float32(0) if Dm == 0 else mn[j] / Dm, 0, 63), (b, j)
            S, M = D * np.float32(F[j]), Dm * np.float32(F[8 + j])
            codes = nibbles(blk[b, 16 + 16 * j:32 + 16 * j])
            for i in range(32):
                t = np.float32(0) if S == 0 else (x[j, i] + M) / S
                assert codes[i] == best_code(t, 0, 15), (b, j, i)


def test_q4_k_error_bound_and_top_codes():
    rng = np.random.default_rng(32)
    w = (rng.standard_normal((8, 1024)) * np.exp(rng.uniform(-6, 0, (8, 1)))).astype(np.float32)
    w[0, :256] = np.abs(w[0, :256])  # a super-block with no negative weight
    b = O.quantize_q4_k(w).reshape(8, -1, 144)
    y = O.dequant(O.Q4_K, b.reshape(-1), 8, 1024).reshape(8, -1, 8, 32)
    for r in range(8):
        for s in range(b.shape[1]):
            D = f16val(int(b[r, s, 0:2].view("<u2")[0]))
            Dm = f16val(int(b[r, s, 2:4].view("<u2")[0]))
            F = q4k_fields(b[r, s, 4:16])
            assert max(F[:8]) == 63  # the widest sub-block takes the top 6-bit code
            x = w[r, 256 * s:256 * s + 256].reshape(8, 32).astype(np.float64)
            if x.min() < 0:
                assert max(F[8:]) == 63
            else:
                assert Dm == 0 and max(F[8:]) == 0
            for j in range(8):
                S = D * F[j]
                bound = S / 2 + 15 * D / 2 + Dm / 2
                err = np.abs(x[j] - y[r, s, j]).max()
                assert err <= bound * (1 + 1e-5) + 1e-30, (r, s, j)


def test_q4_k_degenerate_blocks():
    w = np.zeros((3, 256), dtype=np.float32)
    w[1, :] = np.float32(-0.375)  # constant negative: zero scale, the min carries it
    w[2, :] = np.float32(0.375)   # constant positive: zero min
    b = O.quantize_q4_k(w).reshape(-1, 144)
    assert np.all(b[0] == 0)
    y = O.dequant(O.Q4_K, b.reshape(-1), 3, 256)
    assert np.all(y[0] == 0)
    F1 = q4k_fields(b[1, 4:16])
    assert int(b[1, 0:2].view("<u2")[0]) == 0 and F1[:8] == [0] * 8 and F1[8:] == [63] * 8
    Dm = f16val(int(b[1, 2:4].view("<u2")[0]))
    assert np.all(np.abs(y[1] + 0.375) <= Dm / 2)
    assert np.all(b[1, 16:] == 0)
    F2 = q4k_fields(b[2, 4:16])
    assert int(b[2, 2:4].view("<u2")[0]) == 0 and F2[8:] == [0] * 8
    D = f16val(int(b[2, 0:2].view("<u2")[0]))
    assert np.all(np.abs(y[2] - 0.375) <= D * 63 / 2 * (1 + 1e-6))


# --------------------------------------------------------------------------
# group-128 W4 weights and 8-bit activations (TurboQuant article 2.1, 2.2)
# --------------------------------------------------------------------------
def w4_planes(blocks, rows, k):
    """(codes rows x k/2, fp16 scale bits rows x k/128) of the planar layout (R28)."""
    b = np.asarray(blocks, dtype=np.uint8)
    codes = b[: rows * k // 2].reshape(rows, k // 2)
    scales = b[rows * k // 2:].copy().view("<u2").reshape(rows, k // 128)
    return codes, scales


def test_w4g128_hand_built_planes():
    rows, k = 2, 256
    b = np.zeros(rows * k // 2 + rows * (k // 128) * 2, np.uint8)
    assert b.size == O.packed_bytes(O.W4G128, rows, k) == 2 * 2 * 66
    codes = b[:256].reshape(2, 128)
    codes[0, 0] = 0xF0     # row 0 group 0: weight 0 code 0 (-8), weight 64 code 15 (+7)
    codes[0, 64 + 5] = 0x9A  # row 0 group 1: weight 128+5 code 10 (+2), weight 128+69 code 9 (+1)
    codes[1, :] = 0x88     # row 1: all codes 8 (0)
    codes[1, 127] = 0x08   # row 1 group 1: weight 128+63 code 8, weight 255 code 0 (-8)
    b[256:264] = np.array([0x3800, 0x2400, 0x3C00, 0xBC00], dtype="<u2").view(np.uint8)  # 0.5, 1/64, 1, -1
    y = O.dequant(O.W4G128, b, rows, k)
    assert y[0, 0] == -4.0 and y[0, 64] == 3.5
    assert y[0, 128 + 5] == 2 / 64 and y[0, 128 + 69] == 1 / 64
    assert y[0, 1] == -4.0  # byte 1 is 0x00: codes 0 -> -8 * 0.5
    assert y[1, 191] == 0.0 and y[1, 255] == 8.0  # -1 * -8
    assert np.count_nonzero(y[1]) == 1


def test_brute_force_w4g128_codes():
    rng = np.random.default_rng(25)
    w = tiny_blocks(rng, 12, 128).reshape(3, 512)
    b = O.quantize_w4g128(w)
    codes, scales = w4_planes(b, 3, 512)
    for r in range(3):
        for g in range(4):
            x = w[r, 128 * g:128 * g + 128]
            assert scales[r, g] == f16(np.float32(np.abs(x).max()) / np.float32(7.0))
            d = np.float32(f16val(int(scales[r, g])))
            byte = codes[r, 64 * g:64 * g + 64].astype(np.int64)
            n = np.concatenate([byte & 15, byte >> 4])
            for i in range(128):
                t = np.float32(0.0) if d == 0 else x[i] / d
                assert n[i] - 8 == best_code(t, -8, 7), (r, g, i)


def test_brute_force_act_i8():
    rng = np.random.default_rng(26)
    x = tiny_blocks(rng, 6, 300)
    x[5] = 0.0
    xq, s = O.quantize_act_i8(x)
    for t in range(6):
        assert s[t] == np.float32(np.abs(x[t]).max()) / np.float32(127.0)
        for i in range(300):
            q = np.float32(0.0) if s[t] == 0 else x[t, i] / s[t]
            assert xq[t, i] == best_code(q, -127, 127), (t, i)
        if s[t] > 0:
            assert np.abs(xq[t]).max() == 127  # the largest magnitude takes the top level
    assert np.all(xq[5] == 0)
    # 16-bit inputs read exactly as their fp32 values
    h = x[:5].astype(np.float16)
    xq16, s16 = O.quantize_act_i8(h)
    xq32, s32 = O.quantize_act_i8(h.astype(np.float32))
    assert np.array_equal(xq16, xq32) and np.array_equal(s16, s32)


def test_w4a8_product_is_the_exact_rational_sum():
    # sum over groups of d_g * s_t * (integer dot of codes-8 and xq): exact
    # rationals, against the oracle's fp64 per-element sums
    rng = np.random.default_rng(27)
    m, k, n = 5, 384, 3
    w = (rng.standard_normal((m, k)) * 0.05).astype(np.float32)
    x = rng.standard_normal((n, k)).astype(np.float32)
    b = O.quantize_w4g128(w)
    xq, s = O.quantize_act_i8(x)
    Y, B = O.gemm_w4a8(b, m, k, xq, s)
    codes, scales = w4_planes(b, m, k)
    for i in range(m):
        for t in range(n):
            exact = Fraction(0)
            for g in range(k // 128):
                byte = codes[i, 64 * g:64 * g + 64].astype(np.int64)
                nn = np.concatenate([byte & 15, byte >> 4]) - 8
                dot = int(np.dot(nn, xq[t, 128 * g:128 * g + 128].astype(np.int64)))
                exact += Fraction(f16val(int(scales[i, g]))) * dot
            exact *= Fraction(float(s[t]))
            assert abs(Fraction(float(Y[t, i])) - exact) <= Fraction(1e-15) * Fraction(float(B[t, i]))
    W = O.dequant(O.W4G128, b, m, k).astype(np.float64)
    Xr = s[:, None].astype(np.float64) * xq
    assert np.allclose(Y, Xr @ W.T, rtol=0, atol=1e-12 * B.max())
    rows = np.array([4, 0])
    Y2, _ = O.gemm_w4a8(b, m, k, xq, s, rows=rows)
    assert np.array_equal(Y2, Y[:, rows])


def test_w4g128_idempotent_and_degenerate():
    rng = np.random.default_rng(28)
    w = (rng.standard_normal((4, 1024)) * 0.02).astype(np.float32)
    w[3] = 0.0
    b = O.quantize_w4g128(w)
    b2 = O.quantize_w4g128(O.dequant(O.W4G128, b, 4, 1024))
    assert np.array_equal(b, b2)
    codes, scales = w4_planes(b, 4, 1024)
    assert np.all(codes[3] == 0x88) and np.all(scales[3] == 0)
    y = O.dequant(O.W4G128, b, 4, 1024)
    d = np.repeat(scales.view(np.float16).astype(np.float64), 128, axis=1)
    assert np.all(np.abs(w - y) <= d / 2 * (1 + 2.0 ** -22) + 1e-30)


# --------------------------------------------------------------------------
# the fp64 products, against numpy's float64 matmul
# --------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", [O.Q4_0, O.SB4, O.SB4_AFFINE, O.Q4_K, O.W4G128])
def test_products_vs_numpy(fmt):
    rng = np.random.default_rng(41 + fmt)
    m, k = 24, 768
    w = (rng.standard_normal((m, k)) * 0.02).astype(np.float32)
    b = O.quantize(fmt, w)
    W = O.dequant(fmt, b, m, k).astype(np.float64)
    # a unit vector picks one column, bit for bit
    for col in (0, 257, k - 1):
        e = np.zeros(k)
        e[col] = 1.0
        y, _ = O.gemv(fmt, b, m, k, e)
        assert np.array_equal(y, W[:, col])
    x = rng.standard_normal(k)
    y, bound = O.gemv(fmt, b, m, k, x)
    assert np.allclose(y, W @ x, rtol=0, atol=1e-12 * bound.max())
    assert np.allclose(bound, np.abs(W * x).sum(1))
    rows = np.array([5, 0, 23])
    y2, _ = O.gemv(fmt, b, m, k, x, rows=rows)
    assert np.array_equal(y2, y[rows])
    X = rng.standard_normal((3, k))
    Y, B = O.gemm(fmt, b, m, k, X)
    assert np.allclose(Y, X @ W.T, rtol=0, atol=1e-12 * B.max())
    Y2, _ = O.gemm(fmt, b, m, k, X, rows=rows)
    assert np.array_equal(Y2, Y[:, rows])


def test_oracle_rejects_bad_arguments():
    with pytest.raises(ValueError):
        O.quantize_q4_0(np.zeros((1, 33), np.float32))
    with pytest.raises(ValueError):
        O.quantize_sb4(np.zeros((1, 128), np.float32))
