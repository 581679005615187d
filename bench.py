#!/usr/bin/env python3
"""Benchmark of the block-quantized hot path on one MI355X.

Headline (one JSON line on stdout): batch-1 dequant-GEMV of an 11008 x 4096
super-block Type 0 matrix (138-byte blocks, per-row std log-uniform in
[0.005, 0.05]), x fp16 ~N(0,1), y fp32 -- effective HBM GB/s = algorithmic
bytes (blocks + x + y = 24,357,888 B) / time per GEMV.

A step is one GEMV launch.  The weights rotate through enough distinct copies
(> 2x the 256 MB last-level cache) that every step streams them from HBM.  The
K timed steps are launched eagerly and back to back and timed with HIP
events, the start event queued behind a device-side wait longer than the
host needs to submit them (so the GPU runs them with no host gaps, and
without the fixed ~10 us a HIP graph replay adds); the average launch
duration is the timed region / K.  Beside the nominal 8 TB/s,
"hbm_reference" gives what a plain streaming read of the same bytes (and of
1 GiB) reaches on the same GPU, the launch cost of an empty kernel timed the
same way, and torch's copy.

Also measured (field "rows"): every other step of the hot path at the shapes
of the synthetic workloads -- quantization (Q4_0, super-block Type 0 and
Type 1 over a 32-layer 7B-shaped stack from fp16, Q4_K), dequantization, the
Q4_0, Type 1 and Q4_K GEMVs and the prefill GEMM (N = 16, 64, 512) for every
format.

cpu_baseline: the CPU oracle (oracle/, plain C, fp64 sums) timed on this
host on the same GEMV workload, on one thread and on every core (row chunks).
"""
import argparse
import contextlib
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MALL_BYTES = 256 << 20
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_sb4_11008x4096.json")


def kernel_source_hash():
    """What the headline kernel's machine code comes from: its sources and the
    compiler flags of the build (bit_block_quant_amd/build.py, read by path)."""
    import importlib.util

    h = hashlib.sha256()
    for f in ("qblk_gemv.hip", "qblk_device.h"):
        with open(os.path.join(ROOT, "bit_block_quant_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    spec = importlib.util.spec_from_file_location("_qblk_build_flags",
                                                  os.path.join(ROOT, "bit_block_quant_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    h.update(" ".join(mod.FLAGS).encode())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Timer:
    """Time `launch(i % n)` for i in range(n * rot) (rot passes over the n
    rotating inputs), launched eagerly and back to back: the timed launches
    are queued behind a device-side wait longer than the host needs to
    submit them, so the GPU runs them without host gaps.  (A HIP graph of
    the same launches costs a fixed ~10 us per replay on top: 20 headline
    GEMVs averaged 7.1-7.4 us per launch from a graph, 6.62 us eagerly.)"""

    def __init__(self, torch, launch, n, rot=1):
        self.torch = torch
        self.launch = launch
        self.n_in = n
        self.n = n * rot
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):  # first pass: loads the kernels, measures the host's cost per launch
            launch(i)
        self.host_us = (time.perf_counter() - t0) * 1e6 / n
        torch.cuda.synchronize()

    def pass_(self, count):
        for i in range(count):
            self.launch(i % self.n_in)

    def run(self, reps, warmup=1):
        t = self.torch
        for _ in range(warmup):
            self.pass_(self.n)
        t.cuda.synchronize()
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        with no_gc():
            lead_in(t, 200.0 + 2.0 * self.host_us * reps * self.n)
            a.record()
            for _ in range(reps):
                self.pass_(self.n)
            b.record()
        t.cuda.synchronize()
        return a.elapsed_time(b) / (reps * self.n)  # ms per launch


@contextlib.contextmanager
def no_gc():
    """The interpreter's garbage collector, collected first and then paused
    while a timed region is submitted: a collection in the middle (tens of
    ms) outlasts the lead-in wait and leaves the GPU idle inside the region
    (seen as ~300 us per launch over 120 batched GEMV launches)."""
    gc.collect()
    gc.disable()
    try:
        yield
    finally:
        gc.enable()


def lead_in(torch, us=300.0):
    """Queue a wait of about `us` on the current stream (one wave polling the
    device clock) just before a timed region's start event, so that the
    region starts with its work already queued instead of measuring the
    host's submission as well."""
    import ctypes as Cty
    rc = _hbmref_lib().hbmref_spin(us, Cty.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, rc


def time_region(torch, fn, lead_us=300.0):
    """ms for fn() on the current stream, HIP events, synchronized both sides;
    the region starts after a lead-in wait of lead_us, with fn's work queued."""
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with no_gc():
        lead_in(torch, lead_us)
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b)


_HBMREF = []


def _hbmref_lib():
    """libqblk_hbmref.so: a plain streaming read, an empty kernel and a timed
    wait, built beside libqblk but not part of it."""
    import ctypes as C
    if _HBMREF:
        return _HBMREF[0]
    path = os.path.join(ROOT, "bit_block_quant_amd", "libqblk_hbmref.so")
    L = C.CDLL(path)
    L.hbmref_spin.argtypes, L.hbmref_spin.restype = [C.c_double, C.c_void_p], C.c_int
    _HBMREF.append(L)
    L.hbmref_read.argtypes, L.hbmref_read.restype = [C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p], C.c_int
    L.hbmref_empty.argtypes, L.hbmref_empty.restype = [C.c_uint, C.c_void_p, C.c_void_p], C.c_int
    return L


def hbm_reference(torch, dev, nbytes, C):
    """What the memory system delivers to kernels that only move bytes, beside
    the nominal 8 TB/s: a plain 16-byte-per-thread read of the headline's byte
    count over C rotating buffers (so every launch reads HBM) and of 1 GiB;
    torch's copy kernel over the same (bytes = read + write); and the launch
    cost of an empty kernel of 256 workgroups timed the same way."""
    import ctypes as Cty
    out = {}
    L = _hbmref_lib()
    sink = torch.zeros(64, dtype=torch.int32, device=dev)

    def rec(name, ms, nb):
        gbs = nb / (ms * 1e-3) / 1e9 if nb else 0.0
        out[name] = {"us": round(ms * 1e3, 3), "GBps": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}
        log(f"  reference {name}: {ms * 1e3:.2f} us" + (f", {gbs:.0f} GB/s" if nb else ""))

    def stream_ptr():
        return Cty.c_void_p(torch.cuda.current_stream().cuda_stream)

    for name, nb, n in (("read_24MB_rotating", nbytes, C), ("read_1GiB", 1 << 30, 2)):
        nb16 = nb // 16 * 16
        bufs = [torch.ones(nb16 // 4, dtype=torch.float32, device=dev) for _ in range(n)]

        def launch(i, bufs=bufs, nb16=nb16):
            rc = L.hbmref_read(Cty.c_void_p(bufs[i % len(bufs)].data_ptr()), nb16,
                               Cty.c_void_p(sink.data_ptr()), stream_ptr())
            assert rc == 0, rc
        t = Timer(torch, launch, n, max(1, 480 // n) if nb16 < (1 << 28) else 4)
        rec(name, t.run(2), nb16)
        del bufs
    t = Timer(torch, lambda i: L.hbmref_empty(256, Cty.c_void_p(sink.data_ptr()), stream_ptr()), 480)
    rec("empty_kernel_256wg", t.run(2), 0)
    for name, nb, n in (("copy_24MB_rotating", nbytes, C), ("copy_1GiB", 1 << 30, 1)):
        n_el = nb // 4
        src = [torch.empty(n_el, dtype=torch.float32, device=dev) for _ in range(n)]
        dst = torch.empty(n_el, dtype=torch.float32, device=dev)
        for t in src:
            t.fill_(1.0)
        t = Timer(torch, lambda i: dst.copy_(src[i]), n)
        rec(name, t.run(max(1, 480 // n)), 2 * n_el * 4)
        del src, dst
    return out


def n_copies(nbytes):
    return max(2, -(-2 * MALL_BYTES // nbytes) + 1)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000, help="timed GEMV launches")
    ap.add_argument("--warmup", type=int, default=200, help="untimed GEMV launches")
    ap.add_argument("--rows", type=int, default=1, help="1: also time the other hot-path steps")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU-baseline budget (0: skip)")
    ap.add_argument("--mode", choices=("full", "traffic", "gemm"), default="full",
                    help="traffic: a 256 MiB device copy (counter calibration) then a few "
                         "headline GEMV launches, for rocprofv3 --pmc runs; gemm: three "
                         "launches of one prefill GEMM (--gemm-shape, --gemm-n), for counters")
    ap.add_argument("--gemv-case", choices=tuple(GEMV_CASES), default="sb4_11008x4096",
                    help="decode GEMV of the --mode traffic launches")
    ap.add_argument("--gemm-shape", choices=("up", "down"), default="up")
    ap.add_argument("--gemm-n", type=int, default=512)
    ap.add_argument("--gemm-fmt", choices=("sb4", "q4_0", "sb4a", "q4k", "w4a8"), default="sb4",
                    help="weight format of the --mode gemm launches (w4a8: group-128 weights, int8 tokens)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from __graft_entry__ import _ensure_built
    _ensure_built()
    import bit_block_quant_amd as q
    import workloads as WL

    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    dev = torch.device("cuda:0")

    if args.mode == "traffic":
        traffic_run(torch, q, WL, dev, args.gemv_case)
        return
    if args.mode == "gemm":
        gemm_run(torch, q, WL, np, dev, args.gemm_shape, args.gemm_n, args.gemm_fmt)
        return

    # ------------------------------------------------------------ headline
    w, x = WL.sb4_decode("up")
    M, K = w.shape
    blocks0 = q.quantize(torch.from_numpy(w).to(dev), q.SB4)
    nbytes = blocks0.numel()
    C = n_copies(nbytes)
    copies = [blocks0] + [blocks0.clone() for _ in range(C - 1)]
    xd = torch.from_numpy(x).to(dev)
    yd = torch.empty(M, dtype=torch.float32, device=dev)
    algo_bytes = nbytes + 2 * K + 4 * M
    log(f"gemv sb4 {M}x{K}: {nbytes} B of blocks, {C} rotating copies ({C * nbytes / 2**20:.0f} MiB)")

    # exactly `steps` launches, eager and back to back (see Timer), copy
    # i % C for step i
    launch = lambda i: q.gemv(copies[i % C], q.SB4, M, K, xd, out=yd)  # noqa: E731
    t_first = Timer(torch, launch, C)  # loads the kernel, measures the host's cost per launch
    # untimed warmup launches on the copies the timed region reads last (or
    # not at all), so none of the first timed launches finds its weights
    # still in the 256 MB last-level cache
    for i in range(args.warmup):
        launch((C - args.warmup % C + i) % C)

    def region():
        for i in range(args.steps):
            launch(i)

    steps = args.steps
    ms = time_region(torch, region, 300.0 + 2.0 * t_first.host_us * steps) / steps
    gbs = algo_bytes / (ms * 1e-3) / 1e9
    log(f"  {ms * 1e3:.2f} us per GEMV, {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s)")
    achievable = hbm_reference(torch, dev, nbytes, C)

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        t = json.load(open(TRAFFIC_FILE))
        if t.get("kernel_source_hash") == kernel_source_hash():
            traffic = t.get("bytes_per_launch")

    result = {
        "metric": "dequant-GEMV effective HBM GB/s (% of ~8 TB/s peak), 11008x4096 batch 1",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "sb4_type0_gemv_11008x4096_batch1",
            "format": "super-block Type 0, 138 B per 256 weights",
            "m": M, "k": K, "x": "f16", "y": "f32",
            "algorithmic_bytes": algo_bytes,
            "rotating_copies": C,
            "timing": "back-to-back eager launches queued behind a device-side wait, HIP events",
        },
        "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "roofline": {
            "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
        },
        "hbm_reference": achievable,
        "inputs": {"numpy": WL.NUMPY_VERSION, "w_f32_sha256": WL.sha256(w), "x_f16_sha256": WL.sha256(x),
                   "seeds": WL.SEEDS["sb4_decode_up"]},
        "device": props.name,
        "arch": getattr(props, "gcnArchName", ""),
        "weights_per_s": round(M * K / (ms * 1e-3), 1),
        "gemv_per_s": round(1.0 / (ms * 1e-3), 1),
    }
    del copies

    if args.rows:
        result["rows"] = measure_rows(torch, q, WL, np, dev)

    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(np, WL, w, x, algo_bytes, args.cpu_seconds)
    print(json.dumps(result), flush=True)


# ------------------------------------------------------- counter calibration
CALIB_BYTES = 256 << 20


# decode GEMVs that --mode traffic can run: (format name, workload, x dtype)
GEMV_CASES = {
    "sb4_11008x4096": ("SB4", "sb4_up"),
    "sb4_4096x11008": ("SB4", "sb4_down"),
    "q4_0_4096x4096": ("Q4_0", "q4_0_decode"),
    "sb4a_11008x4096": ("SB4_AFFINE", "sb4_up"),
    "sb4a_4096x11008": ("SB4_AFFINE", "sb4_down"),
    "sb4a_4096x4096": ("SB4_AFFINE", "q4_0_decode"),
}


def traffic_run(torch, q, WL, dev, case="sb4_11008x4096"):
    """A known-size streaming kernel (fp32 multiply: reads and writes
    CALIB_BYTES once each), then 8 launches of one decode GEMV on distinct
    copies of its blocks (every launch reads HBM)."""
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()
    del src, dst
    fmt_name, wl = GEMV_CASES[case]
    fmt = getattr(q, fmt_name)
    if wl == "sb4_up":
        w, x = WL.sb4_decode("up")
    elif wl == "sb4_down":
        w, x = WL.sb4_decode("down")
    else:
        w, x = WL.q4_0_decode()
    M, K = w.shape
    b0 = q.quantize(torch.from_numpy(w).to(dev), fmt)
    C = n_copies(b0.numel())
    cps = [b0] + [b0.clone() for _ in range(C - 1)]
    xd = torch.from_numpy(x).to(dev)
    y = torch.empty(M, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    for i in range(8):
        q.gemv(cps[(i + 1) % C], fmt, M, K, xd, out=y)
    torch.cuda.synchronize()
    log(f"traffic run done ({case})")


def gemm_run(torch, q, WL, np, dev, shape, n_tok, fmt_name="sb4"):
    """Three launches of one prefill GEMM on the seeded workload (one weight
    copy: for counter runs, not timing)."""
    w, X = WL.sb4_prefill(shape, n_tok)
    m, k = w.shape
    fmt = {"sb4": q.SB4, "q4_0": q.Q4_0, "sb4a": q.SB4_AFFINE, "q4k": q.Q4_K, "w4a8": q.W4G128}[fmt_name]
    b = q.quantize(torch.from_numpy(w).to(dev), fmt)
    Xd = torch.from_numpy(X.view(np.int16)).to(dev).view(torch.bfloat16)
    Y = torch.empty((n_tok, m), dtype=torch.float32, device=dev)
    if fmt == q.W4G128:
        xq, xs = q.quantize_act_i8(Xd)
        run = lambda: q.gemm_w4a8(b, m, k, xq, xs, out=Y)  # noqa: E731
    else:
        run = lambda: q.gemm(b, fmt, m, k, Xd, out=Y)  # noqa: E731
    torch.cuda.synchronize()
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    log(f"gemm run done ({fmt_name}, {shape}, {m}x{k}, n={n_tok})")


# ----------------------------------------------------------------- other rows
def measure_rows(torch, q, WL, np, dev):
    rows = {}
    gen = torch.Generator(device=dev)

    def randn(shape, std, seed, dtype=torch.float32):
        gen.manual_seed(seed)
        t = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
        return (t * std).to(dtype)

    def hbm_row(name, ms, nbytes, **extra):
        gbs = nbytes / (ms * 1e-3) / 1e9
        rows[name] = dict(us=round(ms * 1e3, 3), bytes=nbytes, GBps=round(gbs, 1),
                          frac_hbm=round(gbs / HBM_PEAK_GBS, 4), **extra)
        log(f"  {name}: {ms * 1e3:.2f} us, {gbs:.0f} GB/s")

    # GEMVs with rotation
    def gemv_row(name, fmt, w, x):
        m, k = w.shape
        b0 = q.quantize(w, fmt)
        C = n_copies(b0.numel())
        cps = [b0] + [b0.clone() for _ in range(C - 1)]
        y = torch.empty(m, dtype=torch.float32, device=dev)
        t = Timer(torch, lambda i: q.gemv(cps[i], fmt, m, k, x, out=y), C, max(1, 400 // C))
        ms = t.run(1)
        # the plain 16-byte read of the same blocks, timed the same way: what a
        # kernel that only reads them reaches at this size
        import ctypes as Cty
        L = _hbmref_lib()
        sink = torch.zeros(64, dtype=torch.int32, device=dev)
        nb16 = b0.numel() // 16 * 16
        tr = Timer(torch, lambda i: L.hbmref_read(Cty.c_void_p(cps[i].data_ptr()), nb16, Cty.c_void_p(sink.data_ptr()),
                                                  Cty.c_void_p(torch.cuda.current_stream().cuda_stream)),
                   C, max(1, 400 // C))
        read_ms = tr.run(1)
        hbm_row(name, ms, b0.numel() + x.numel() * x.element_size() + 4 * m, m=m, k=k,
                read_ref_us=round(read_ms * 1e3, 3), read_ref_over_gemv=round(read_ms / ms, 3))

    w, x = WL.sb4_decode("down")
    gemv_row("gemv_sb4_4096x11008_f16", q.SB4, torch.from_numpy(w).to(dev), torch.from_numpy(x).to(dev))
    w, x = WL.q4_0_decode()
    gemv_row("gemv_q4_0_4096x4096_f16", q.Q4_0, torch.from_numpy(w).to(dev), torch.from_numpy(x).to(dev))
    w, x = WL.q4_0_small()
    gemv_row("gemv_q4_0_256x4096_f32", q.Q4_0, torch.from_numpy(w).to(dev), torch.from_numpy(x).to(dev))
    w, x = WL.sb4_decode("up")
    gemv_row("gemv_q4k_11008x4096_f16", q.Q4_K, torch.from_numpy(w).to(dev), torch.from_numpy(x).to(dev))
    # the prefill workload's 14336x4096 Type 0 matrix (gate/up of an 8B
    # model) at batch 1, with the decode workload's x
    w14, _ = WL.sb4_prefill("up", 1)
    gemv_row("gemv_sb4_14336x4096_f16", q.SB4, torch.from_numpy(w14).to(dev), torch.from_numpy(x).to(dev))
    del w14

    # the headline matrix as a layer's gate and up projections: two 11008x4096
    # Type 0 matrices against one x in one qblk_gemv_batch launch (pairs of
    # rotating copies, cold in the last-level cache)
    wt, xt_ = torch.from_numpy(w).to(dev), torch.from_numpy(x).to(dev)
    b0 = q.quantize(wt, q.SB4)
    m, k = wt.shape
    C = n_copies(2 * b0.numel())
    cps = [b0] + [b0.clone() for _ in range(2 * C - 1)]
    ys2 = [torch.empty(m, dtype=torch.float32, device=dev) for _ in range(2)]
    t = Timer(torch, lambda i: q.gemv_batch(q.SB4, k, [(cps[2 * i], m, xt_), (cps[2 * i + 1], m, xt_)], outs=ys2),
              C, max(1, 200 // C))
    ms = t.run(1)
    hbm_row("gemv_sb4_11008x4096x2_f16_batched", ms, 2 * (b0.numel() + xt_.numel() * 2 + 4 * m), matrices=2,
            us_per_matrix=round(ms * 1e3 / 2, 3))
    del cps, wt, b0

    # quantizers
    def quant_row(name, fmt, w):
        # rotating input copies (past the last-level cache), C launches per pass
        out = torch.empty(q.packed_bytes(fmt, *w.shape), dtype=torch.uint8, device=dev)
        C = n_copies(w.numel() * w.element_size())
        ws = [w] + [w.clone() for _ in range(C - 1)]
        t = Timer(torch, lambda i: q.quantize(ws[i], fmt, out=out), C)
        ms = t.run(max(2, 40 // C))
        nb = w.numel() * w.element_size() + out.numel()
        hbm_row(name, ms, nb, weights_per_s=round(w.numel() / (ms * 1e-3), 1))
        del ws

    w, _ = WL.q4_0_decode()
    quant_row("quantize_q4_0_4096x4096_f32", q.Q4_0, torch.from_numpy(w).to(dev))
    w, _ = WL.sb4_decode("up")
    wup = torch.from_numpy(w).to(dev)
    quant_row("quantize_sb4_11008x4096_f32", q.SB4, wup)
    quant_row("quantize_sb4a_11008x4096_f32", q.SB4_AFFINE, wup)
    quant_row("quantize_q4k_11008x4096_f32", q.Q4_K, wup)
    quant_row("quantize_q4k_11008x4096_f16", q.Q4_K, wup.half())

    # dequant
    b = q.quantize(wup, q.SB4)
    out = torch.empty(wup.shape, dtype=torch.float32, device=dev)
    C = n_copies(b.numel())
    bs = [b] + [b.clone() for _ in range(C - 1)]
    t = Timer(torch, lambda i: q.dequant(bs[i], q.SB4, *wup.shape, out=out), C)
    hbm_row("dequant_sb4_11008x4096_to_f32", t.run(max(2, 120 // C)), b.numel() + out.numel() * 4)
    del wup, out, b, bs

    # 7B-shaped 32-layer stack, Type 1: quantize from fp16, then one GEMV pass
    mats, outs, xs = [], [], []
    for layer in range(WL.STACK_LAYERS):
        for p, (_, r, k) in enumerate(WL.STACK_PROJ):
            sw, sx = WL.stack_seed(layer, p)
            mats.append(randn((r, k), 0.02, sw, torch.float16))
            outs.append(torch.empty(q.packed_bytes(q.SB4_AFFINE, r, k), dtype=torch.uint8, device=dev))
            xs.append(randn((k,), 1.0, sx, torch.float16))
    n = len(mats)
    # the stack is drawn on the device with torch's generator (the numpy recipe
    # would take minutes on the host for 6.5e9 weights); its fingerprint: the
    # SHA-256 over the first 65536 values of every matrix and every x, in order
    fp = hashlib.sha256()
    for mt, xx in zip(mats, xs):
        fp.update(mt.reshape(-1)[:65536].cpu().numpy().tobytes())
        fp.update(xx.reshape(-1)[:65536].cpu().numpy().tobytes())
    stack_inputs = {"generator": f"torch {torch.__version__} default CUDA generator, manual_seed per matrix",
                    "sha256_first64k_each": fp.hexdigest()}
    t = Timer(torch, lambda i: q.quantize(mats[i], q.SB4_AFFINE, out=outs[i]), n)
    ms = t.run(2) * n
    src = sum(m.numel() * 2 for m in mats)
    dst = sum(o.numel() for o in outs)
    hbm_row("quantize_sb4a_stack_32x7_f16", ms, src + dst,
            weights=sum(m.numel() for m in mats), weights_per_s=round(sum(m.numel() for m in mats) / (ms * 1e-3), 1),
            inputs=stack_inputs)
    del mats
    ys = [torch.empty(WL.STACK_PROJ[i % 7][1], dtype=torch.float32, device=dev) for i in range(n)]

    def stack_gemv(i):
        _, r, k = WL.STACK_PROJ[i % 7]
        q.gemv(outs[i], q.SB4_AFFINE, r, k, xs[i], out=ys[i])

    t = Timer(torch, stack_gemv, n)
    ms = t.run(3) * n
    nb = dst + sum(xx.numel() * 2 for xx in xs) + sum(yy.numel() * 4 for yy in ys)
    hbm_row("gemv_sb4a_stack_32x7_f16", ms, nb, tokens_per_s_equivalent=round(1.0 / (ms * 1e-3), 1),
            inputs=stack_inputs)

    # the same pass with each layer's matrices of equal k in one qblk_gemv_batch
    # call (k = 4096: q, k, v, o, gate, up; k = 11008: down): 2 launches a layer
    groups = []
    for layer in range(WL.STACK_LAYERS):
        by_k = {}
        for p, (_, r, k) in enumerate(WL.STACK_PROJ):
            by_k.setdefault(k, []).append(layer * len(WL.STACK_PROJ) + p)
        for k, idx in by_k.items():
            groups.append((k, [(outs[i], WL.STACK_PROJ[i % 7][1], xs[i]) for i in idx], [ys[i] for i in idx]))

    def stack_batch(g):
        k, prods, yo = groups[g]
        q.gemv_batch(q.SB4_AFFINE, k, prods, outs=yo)

    t = Timer(torch, stack_batch, len(groups))
    ms = t.run(3) * len(groups)
    hbm_row("gemv_sb4a_stack_32x7_f16_batched", ms, nb, launches=len(groups),
            tokens_per_s_equivalent=round(1.0 / (ms * 1e-3), 1), inputs=stack_inputs)
    del outs, xs, ys, groups

    # prefill GEMM
    for shape in ("up", "down"):
        w, _ = WL.sb4_prefill(shape, 16)
        m, k = w.shape
        w_sha = WL.sha256(w)
        b0 = q.quantize(torch.from_numpy(w).to(dev), q.SB4)
        C = n_copies(b0.numel())
        cps = [b0] + [b0.clone() for _ in range(C - 1)]
        for n_tok in (16, 64, 512):
            _, X = WL.sb4_prefill(shape, n_tok)
            Xd = torch.from_numpy(X.view(np.int16)).to(dev).view(torch.bfloat16)
            Y = torch.empty((n_tok, m), dtype=torch.float32, device=dev)
            t = Timer(torch, lambda i: q.gemm(cps[i], q.SB4, m, k, Xd, out=Y), C)
            ms = t.run(max(1, 100 // C))
            flops = 2.0 * m * k * n_tok
            nb = b0.numel() + X.size * 2 + Y.numel() * 4
            tf = flops / (ms * 1e-3) / 1e12
            gbs = nb / (ms * 1e-3) / 1e9
            name = f"gemm_sb4_{m}x{k}_n{n_tok}_bf16"
            rows[name] = dict(us=round(ms * 1e3, 3), bytes=nb, GBps=round(gbs, 1),
                              frac_hbm=round(gbs / HBM_PEAK_GBS, 4), TFLOPs=round(tf, 2),
                              frac_mfma_bf16=round(tf / BF16_PEAK_TFLOPS, 4),
                              inputs={"w_f32_sha256": w_sha, "x_bf16_sha256": WL.sha256(X)})
            log(f"  {name}: {ms * 1e3:.2f} us, {gbs:.0f} GB/s, {tf:.1f} TFLOP/s")
        del cps
    # the same product for the other formats (14336x4096)
    w, _ = WL.sb4_prefill("up", 16)
    m, k = w.shape
    wd = torch.from_numpy(w).to(dev)
    for fmt, tag in ((q.Q4_0, "q4_0"), (q.SB4_AFFINE, "sb4a"), (q.Q4_K, "q4k")):
        b0 = q.quantize(wd, fmt)
        C = n_copies(b0.numel())
        cps = [b0] + [b0.clone() for _ in range(C - 1)]
        for n_tok in (16, 64, 512):
            _, X = WL.sb4_prefill("up", n_tok)
            Xd = torch.from_numpy(X.view(np.int16)).to(dev).view(torch.bfloat16)
            Y = torch.empty((n_tok, m), dtype=torch.float32, device=dev)
            t = Timer(torch, lambda i: q.gemm(cps[i], fmt, m, k, Xd, out=Y), C)
            ms = t.run(max(1, 100 // C))
            flops = 2.0 * m * k * n_tok
            nb = b0.numel() + X.size * 2 + Y.numel() * 4
            tf = flops / (ms * 1e-3) / 1e12
            gbs = nb / (ms * 1e-3) / 1e9
            name = f"gemm_{tag}_{m}x{k}_n{n_tok}_bf16"
            rows[name] = dict(us=round(ms * 1e3, 3), bytes=nb, GBps=round(gbs, 1),
                              frac_hbm=round(gbs / HBM_PEAK_GBS, 4), TFLOPs=round(tf, 2),
                              frac_mfma_bf16=round(tf / BF16_PEAK_TFLOPS, 4))
            log(f"  {name}: {ms * 1e3:.2f} us, {gbs:.0f} GB/s, {tf:.1f} TFLOP/s")
        del cps

    # group-128 W4 weights with 8-bit activations
    rows.update(w4a8_rows(torch, q, WL, np, dev))
    return rows


INT8_PEAK_TOPS = 5000.0


def w4a8_rows(torch, q, WL, np, dev):
    rows = {}

    def row(name, ms, nbytes, ops=None):
        gbs = nbytes / (ms * 1e-3) / 1e9
        r = dict(us=round(ms * 1e3, 3), bytes=nbytes, GBps=round(gbs, 1), frac_hbm=round(gbs / HBM_PEAK_GBS, 4))
        msg = f"  {name}: {ms * 1e3:.2f} us, {gbs:.0f} GB/s"
        if ops:
            tops = ops / (ms * 1e-3) / 1e12
            r.update(TOPs=round(tops, 2), frac_mfma_int8=round(tops / INT8_PEAK_TOPS, 4))
            msg += f", {tops:.1f} TOP/s"
        rows[name] = r
        log(msg)

    # weight quantization and one-token product at the decode shape
    w, x = WL.sb4_decode("up")
    m, k = w.shape
    wd = torch.from_numpy(w).to(dev)
    out = torch.empty(q.packed_bytes(q.W4G128, m, k), dtype=torch.uint8, device=dev)
    C = n_copies(wd.numel() * 4)
    ws = [wd] + [wd.clone() for _ in range(C - 1)]
    t = Timer(torch, lambda i: q.quantize(ws[i], q.W4G128, out=out), C)
    row(f"quantize_w4g128_{m}x{k}_f32", t.run(max(2, 40 // C)), wd.numel() * 4 + out.numel())
    b0 = out.clone()
    del wd, out, ws
    xd = torch.from_numpy(x).to(dev).view(1, k)
    xq, xs = q.quantize_act_i8(xd)
    C = n_copies(b0.numel())
    cps = [b0] + [b0.clone() for _ in range(C - 1)]
    y = torch.empty((1, m), dtype=torch.float32, device=dev)
    t = Timer(torch, lambda i: q.gemm_w4a8(cps[i], m, k, xq, xs, out=y), C, max(1, 400 // C))
    row(f"gemv_w4a8_{m}x{k}_i8", t.run(1), b0.numel() + k + 4 + 4 * m)
    t = Timer(torch, lambda i: q.quantize_act_i8(xd, out=xq, scale=xs), 50)  # 50 launches per pass
    row(f"quantize_act_i8_1x{k}_f16", t.run(4), k * 2 + k + 4)
    del cps

    # prefill shape: int8 activations from bf16, then the product
    w, _ = WL.sb4_prefill("up", 16)
    m, k = w.shape
    b0 = q.quantize(torch.from_numpy(w).to(dev), q.W4G128)
    C = n_copies(b0.numel())
    cps = [b0] + [b0.clone() for _ in range(C - 1)]
    for n_tok in (16, 64, 512):
        _, X = WL.sb4_prefill("up", n_tok)
        Xd = torch.from_numpy(X.view(np.int16)).to(dev).view(torch.bfloat16)
        xq, xs = q.quantize_act_i8(Xd)
        if n_tok == 512:
            t = Timer(torch, lambda i: q.quantize_act_i8(Xd, out=xq, scale=xs), 50)
            row(f"quantize_act_i8_{n_tok}x{k}_bf16", t.run(4), n_tok * k * 3 + 4 * n_tok)
        Y = torch.empty((n_tok, m), dtype=torch.float32, device=dev)
        t = Timer(torch, lambda i: q.gemm_w4a8(cps[i], m, k, xq, xs, out=Y), C)
        row(f"gemm_w4a8_{m}x{k}_n{n_tok}_i8", t.run(max(1, 100 // C)),
            b0.numel() + n_tok * k + 4 * n_tok + 4 * n_tok * m, ops=2.0 * m * k * n_tok)
    del cps
    return rows


# --------------------------------------------------------------- CPU oracle
def cpu_threads():
    """Threads for the all-cores legs: the CPUs this process may run on, but no
    more than the box's share per GPU, which it states in OMP_NUM_THREADS (16
    for one GPU on the GPU machines); more workers than that share would oversubscribe it."""
    n = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS")
    if share and share.isdigit() and int(share) > 0:
        n = min(n, int(share))
    return max(1, n)


def cpu_baseline(np, WL, w, x, algo_bytes, budget_s):
    """The oracle (plain C: per-row fp32 dequant, fp64 sums; scalar
    quantizers) on this host, on the same workloads: the headline GEMV (the
    `value`), and the Type 0 / Type 1 quantizers of the same 11008 x 4096
    matrix and the 16-token prefill GEMM at 14336 x 4096 ("legs").  Each leg is
    timed on one thread and on every allowed core (row chunks on a thread
    pool; the C oracle runs with the GIL released)."""
    import oracle as O
    from concurrent.futures import ThreadPoolExecutor

    threads = cpu_threads()
    pool = ThreadPoolExecutor(threads)

    def chunks(m):
        step = (m + threads - 1) // threads
        return [np.arange(r0, min(m, r0 + step), dtype=np.int64) for r0 in range(0, m, step)]

    def timed(fn, budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget or reps >= 1000:
                return el / reps, reps

    leg_budget = budget_s / 8
    m, k = w.shape
    # headline GEMV (the oracle quantizes its own input, untimed)
    blocks = O.quantize_sb4(w)
    xd = x.astype(np.float64)
    ck = chunks(m)
    g1, r1 = timed(lambda: O.gemv(O.SB4, blocks, m, k, xd), 2 * leg_budget)
    gt, rt = timed(lambda: list(pool.map(lambda rows: O.gemv(O.SB4, blocks, m, k, xd, rows=rows), ck)), 2 * leg_budget)
    legs = {}

    # quantizers of the same matrix (f32 in): one thread on a 1024-row slice, all cores on the whole matrix
    for name, affine in (("quantize_sb4_11008x4096_f32", False), ("quantize_sb4a_11008x4096_f32", True)):
        fmt = O.SB4_AFFINE if affine else O.SB4
        nb_out = O.packed_bytes(fmt, m, k)
        s1, _ = timed(lambda: O.quantize_sb4(w[:1024], affine=affine), leg_budget)
        s1 *= m / 1024
        sl = [w[r[0]:r[-1] + 1] for r in ck]
        st, _ = timed(lambda: list(pool.map(lambda a: O.quantize_sb4(a, affine=affine), sl)), leg_budget)
        nb = w.nbytes + nb_out
        legs[name] = {"GBps": round(nb / st / 1e9, 3), "weights_per_s": round(m * k / st, 1),
                      "single_thread_GBps": round(nb / s1 / 1e9, 3), "ms": round(st * 1e3, 2)}
    # 16-token prefill product
    wp, X = WL.sb4_prefill("up", 16)
    mp, kp = wp.shape
    bp = O.quantize_sb4(wp)
    Xv = WL.bf16_values(X).astype(np.float64)
    ckp = chunks(mp)
    p1, _ = timed(lambda: O.gemm(O.SB4, bp, mp, kp, Xv, rows=np.arange(512, dtype=np.int64)), leg_budget)
    p1 *= mp / 512
    pt, _ = timed(lambda: list(pool.map(lambda rows: O.gemm(O.SB4, bp, mp, kp, Xv, rows=rows), ckp)), leg_budget)
    nbp = bp.nbytes + X.size * 2 + 16 * mp * 4
    legs[f"gemm_sb4_{mp}x{kp}_n16"] = {"GBps": round(nbp / pt / 1e9, 3),
                                      "GFLOPs": round(2.0 * mp * kp * 16 / pt / 1e9, 2),
                                      "single_thread_GBps": round(nbp / p1 / 1e9, 3), "ms": round(pt * 1e3, 2)}
    pool.shutdown()
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), cpu)
    except OSError:
        pass
    return {
        "value": round(algo_bytes / gt / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"full {m}x{k} super-block GEMVs (C oracle: per-row fp32 dequant, fp64 sums); "
                  f"{rt} on {threads} threads ({gt * 1e3:.1f} ms each), "
                  f"{r1} on 1 thread ({g1 * 1e3:.1f} ms each); legs: the quantizers of the same matrix "
                  f"(one thread on 1024 rows, scaled) and the 16-token GEMM at {mp}x{kp} (one thread on 512 rows)",
        "single_thread": {"value": round(algo_bytes / g1 / 1e9, 3), "unit": "GB/s", "cores": 1},
        "legs": legs,
        "host_cpu": cpu,
        "threads_rule": "allowed CPUs, at most OMP_NUM_THREADS (the host's CPU share per GPU)",
    }


if __name__ == "__main__":
    main()
