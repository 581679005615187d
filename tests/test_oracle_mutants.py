"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of the oracle's C source -- a dropped
clamp, a flipped tie rule, division where a step multiplies by a reciprocal,
a wrong rounding -- compiles the copy with the oracle's own flags into a
temporary library, and checks that the hand-derived fixtures (the pages'
worked examples and the hand-built blocks under tests/golden/) tell it apart
from the oracle as committed.  The mistakes live only in the temporary copy."""
import ast
import ctypes as C
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "qblk_oracle.c")
GOLDEN = os.path.join(ROOT, "tests", "golden")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")


def _golden_raw(name):
    vals = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                key, _, rest = line.partition("=")
                vals[key.strip()] = rest.strip()
    return vals


def _build(tmp_path, src_text, tag):
    from oracle import build as ob
    c = tmp_path / f"oracle_{tag}.c"
    c.write_text(src_text, encoding="utf-8")
    lib = tmp_path / f"liboracle_{tag}.so"
    cmd = ["gcc", *ob.CFLAGS, str(c), "-I", os.path.join(ROOT, "oracle"), "-o", str(lib), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    L = C.CDLL(str(lib))
    L.orc_quantize_q4_0_ref.argtypes = [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p]
    L.orc_quantize_q4_0_ref.restype = C.c_int
    L.orc_quantize_sb4.argtypes = [C.c_void_p, C.c_int, C.c_int64, C.c_int64, C.c_int, C.c_void_p]
    L.orc_quantize_sb4.restype = C.c_int
    return L


def _listing_bytes(L, w):
    out = np.zeros(18 * (w.size // 32), dtype=np.uint8)
    assert L.orc_quantize_q4_0_ref(w.ctypes.data, w.shape[0], w.shape[1], out.ctypes.data) == 0
    return out.tobytes()


def _listing_fixture_outputs(L):
    """(outputs, expected) for the three hand-built listing blocks."""
    g = _golden_raw("q4_0_listing_cap_and_ties.txt")
    got, want = [], []
    for name in ("cap", "first"):
        w = np.zeros((1, 32), dtype=np.float32)
        for i, v in ast.literal_eval(g[f"{name}_values"]).items():
            w[0, i] = v
        got.append(_listing_bytes(L, w))
        want.append(bytes.fromhex(g[f"{name}_bytes"].replace(" ", "")))
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, 0] = np.array([int(g["recip_e_bits"], 16)], np.uint32).view(np.float32)[0]
    w[0, 7] = np.array([int(g["recip_x_bits"], 16)], np.uint32).view(np.float32)[0]
    b = _listing_bytes(L, w)
    got.append(b[2 + 7] & 0x0F)  # code of weight 7 (low nibble of byte 7)
    want.append(int(g["recip_code_x"]))
    return got, want


def _worked_example_codes(L):
    """The K-quants blog's worked example: the eight INT8 codes of a super-block
    whose sub-block scales are the page's eight values."""
    vals = [0.10, 0.14, 0.11, 0.18, 0.08, 0.16, 0.13, 0.09]
    w = np.zeros((1, 256), dtype=np.float32)
    rng = np.random.default_rng(9)
    for j, v in enumerate(vals):
        sj = np.float32(np.float16(v))
        w[0, 32 * j:32 * j + 32] = rng.uniform(-6, 6, 32).astype(np.float32) * sj
        w[0, 32 * j + 5] = np.float32(7.0) * sj
    out = np.zeros(138, dtype=np.uint8)
    assert L.orc_quantize_sb4(w.ctypes.data, 0, 1, 256, 0, out.ctypes.data) == 0
    return int(out[0:2].view("<u2")[0]), [int(c) for c in out[2:10].view(np.int8)]


WORKED_EXAMPLE = (0x15CF, [70, 99, 78, 127, 56, 113, 92, 63])  # the page's codes; S16 = h(0.18/127)

MUTANTS = [
    # (tag, text replaced, replacement, fixture that must catch it)
    ("no_cap", "n[i] = (uint8_t)(c < 15 ? c : 15);", "n[i] = (uint8_t)c;", "listing"),
    ("last_extreme_wins", "if (fabsf(x[i]) > amax) {", "if (fabsf(x[i]) >= amax) {", "listing"),
    ("divide_not_reciprocal", "float t = x[i] * inv + 8.5f;",
     "float t = (inv != 0.0f ? x[i] / d : 0.0f) + 8.5f;", "listing"),
    ("codes_against_unrounded_super_scale", "Su = orc_f16_to_f32(Sb);", "Su = S;", "worked_example"),
    ("super_scale_over_255_levels", "float S = (d - (-d)) / (float)(hi - lo);",
     "float S = (d - (-d)) / (float)(hi - lo + 1);", "worked_example"),
]


def _fixture(L, pin):
    if pin == "listing":
        return _listing_fixture_outputs(L)
    return _worked_example_codes(L), WORKED_EXAMPLE


@pytest.mark.parametrize("tag,old,new,pin", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, tag, old, new, pin):
    src = open(SRC, encoding="utf-8").read()
    assert src.count(old) == 1, f"the mutation site of {tag} is not unique in the oracle source"
    got, want = _fixture(_build(tmp_path, src, "good"), pin)
    assert got == want, "the committed oracle must match the fixtures"
    got, want = _fixture(_build(tmp_path, src.replace(old, new), tag), pin)
    assert got != want, f"mutant {tag} passes the {pin} fixture"
