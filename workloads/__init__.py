"""Seeded synthetic inputs shaped like the decode/prefill workloads.

This module only draws random numbers (numpy PCG64 via default_rng); it holds
none of the quantization arithmetic.  Both the GPU path's tests/benchmark and
the CPU oracle consume the same host buffers produced here.

Workload recipes (std means standard deviation):
  q4_0_small    256 x 4096 f32 weights ~N(0, 0.02), exactly round(1% of M*K)
                distinct entries multiplied by 10 (outliers); x f32 ~N(0,1).
  q4_0_decode   4096 x 4096, same recipe; x f16 ~N(0,1).
  sb4_decode    11008 x 4096 (gate/up-like) and 4096 x 11008 (down-like);
                row r ~N(0, s_r) with s_r log-uniform in [0.005, 0.05];
                x f16 ~N(0,1).
  sb4a_stack    32 layers x {q,k,v,o: 4096x4096; gate, up: 11008x4096;
                down: 4096x11008}, f16 weights ~N(0, 0.02); x f16 ~N(0,1).
  sb4_prefill   14336 x 4096 and 4096 x 14336 f32 ~N(0, 0.02); activations
                bf16 N x K ~N(0,1), N in {16, 64, 512}.
"""
import hashlib

import numpy as np

NUMPY_VERSION = np.__version__


def sha256(a):
    """SHA-256 (hex) of an array's bytes in C order: the fingerprint recorded
    with every measurement, so a run can show which inputs it used."""
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


# ---------------------------------------------------------------- seeds
SEEDS = {
    "q4_0_small": dict(w=100, outliers=101, x=102),
    "q4_0_decode": dict(w=110, outliers=111, x=112),
    "sb4_decode_up": dict(sigma=120, w=121, x=122),
    "sb4_decode_down": dict(sigma=125, w=126, x=127),
    "sb4_prefill_up": dict(w=140),
    "sb4_prefill_down": dict(w=141),
}

STACK_LAYERS = 32
# (name, rows, k) of the seven projections of one layer
STACK_PROJ = (
    ("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
    ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008),
)


def _rng(seed):
    return np.random.default_rng(seed)


def normal(shape, std, seed, dtype=np.float32):
    """~N(0, std) drawn in float32 and cast to dtype (float32/float16)."""
    a = _rng(seed).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a.astype(dtype, copy=False)


def with_outliers(rows, k, std, seed_w, seed_out, frac=0.01, factor=10.0):
    """Gaussian weights with exactly round(frac*rows*k) distinct entries x factor."""
    w = normal((rows, k), std, seed_w)
    n_out = int(round(frac * rows * k))
    idx = _rng(seed_out).choice(rows * k, size=n_out, replace=False)
    w.reshape(-1)[idx] *= np.float32(factor)
    return w


def per_row_std(rows, k, seed_sigma, seed_w, lo=0.005, hi=0.05):
    """Row r ~N(0, s_r), s_r = exp(U(ln lo, ln hi))."""
    s = np.exp(_rng(seed_sigma).uniform(np.log(lo), np.log(hi), size=rows)).astype(np.float32)
    w = normal((rows, k), 1.0, seed_w)
    w *= s[:, None]
    return w


def bf16_bits(a):
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    return ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)


def bf16_values(bits):
    """bfloat16 bit patterns -> the exact float32 values they hold."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------ workloads
def q4_0_small():
    s = SEEDS["q4_0_small"]
    w = with_outliers(256, 4096, 0.02, s["w"], s["outliers"])
    x = normal((4096,), 1.0, s["x"], np.float32)
    return w, x


def q4_0_decode():
    s = SEEDS["q4_0_decode"]
    w = with_outliers(4096, 4096, 0.02, s["w"], s["outliers"])
    x = normal((4096,), 1.0, s["x"], np.float16)
    return w, x


def sb4_decode(shape="up"):
    """shape 'up': 11008 x 4096; 'down': 4096 x 11008."""
    s = SEEDS["sb4_decode_" + shape]
    rows, k = (11008, 4096) if shape == "up" else (4096, 11008)
    w = per_row_std(rows, k, s["sigma"], s["w"])
    x = normal((k,), 1.0, s["x"], np.float16)
    return w, x


def stack_seed(layer, proj_index):
    return 1000 + 16 * layer + proj_index, 2000 + 16 * layer + proj_index


def sb4a_stack_matrix(layer, proj_index):
    name, rows, k = STACK_PROJ[proj_index]
    sw, sx = stack_seed(layer, proj_index)
    w = normal((rows, k), 0.02, sw, np.float16)
    x = normal((k,), 1.0, sx, np.float16)
    return w, x


def sb4_prefill(shape="up", n=16):
    s = SEEDS["sb4_prefill_" + shape]
    rows, k = (14336, 4096) if shape == "up" else (4096, 14336)
    w = normal((rows, k), 0.02, s["w"])
    X = bf16_bits(normal((n, k), 1.0, 142 + n))
    return w, X
