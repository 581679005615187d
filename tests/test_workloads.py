"""The seeded generators (workloads/) are deterministic and shaped as the
recipes state; no GPU is involved.  The fingerprints a benchmark run records
come from workloads.sha256."""
import numpy as np

import workloads as WL


def test_generators_are_deterministic():
    a, xa = WL.q4_0_small()
    b, xb = WL.q4_0_small()
    assert WL.sha256(a) == WL.sha256(b) and WL.sha256(xa) == WL.sha256(xb)
    assert a.shape == (256, 4096) and a.dtype == np.float32 and xa.dtype == np.float32
    w, X = WL.sb4_prefill("up", 16)
    assert w.shape == (14336, 4096) and X.shape == (16, 4096) and X.dtype == np.uint16


def test_outlier_count_and_row_scales():
    w, _ = WL.q4_0_small()
    s = WL.SEEDS["q4_0_small"]
    base = WL.normal(w.shape, 0.02, s["w"])  # the same draws before the x10 entries
    changed = w != base
    assert int(changed.sum()) == round(0.01 * w.size)
    assert np.array_equal(w[changed], base[changed] * np.float32(10.0))
    w, x = WL.sb4_decode("up")
    assert w.shape == (11008, 4096) and x.dtype == np.float16
    sd = w.std(axis=1)
    assert sd.min() > 0.004 and sd.max() < 0.06  # log-uniform in [0.005, 0.05]


def test_sha256_tracks_content():
    a = np.arange(16, dtype=np.float32)
    b = a.copy()
    b[3] = np.nextafter(b[3], np.float32(np.inf))
    assert WL.sha256(a) != WL.sha256(b)
    assert WL.sha256(a) == WL.sha256(a.reshape(4, 4))
