#!/usr/bin/env python3
"""Benchmark of the block-quantized hot path on one MI355X.

Headline (one JSON line on stdout): batch-1 dequant-GEMV of an 11008 x 4096
super-block Type 0 matrix (138-byte blocks, per-row std log-uniform in
[0.005, 0.05]), x fp16 ~N(0,1), y fp32 -- effective HBM GB/s = algorithmic
bytes (blocks + x + y = 24,357,888 B) / time per GEMV.

A step is one GEMV launch.  The weights rotate through enough distinct copies
(> 2x the 256 MB last-level cache) that every step streams them from HBM.  The
K timed steps are captured in HIP graphs (no host launch gaps) and timed with
HIP events on the replay stream; the average launch duration is the timed
region / K.  Beside the nominal 8 TB/s, "hbm_reference" gives what torch's
plain device copy reaches on the same GPU.

Also measured (field "rows"): every other step of the hot path at the shapes
of the synthetic workloads -- quantization (Q4_0, super-block Type 0 and
Type 1 over a 32-layer 7B-shaped stack from fp16, Q4_K), dequantization, the
Q4_0, Type 1 and Q4_K GEMVs and the prefill GEMM (N = 16, 64, 512) for every
format.

cpu_baseline: the CPU oracle (oracle/, plain C, fp64 sums) timed on this
host on the same GEMV workload, on one thread and on every core (row chunks).
"""
import argparse
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
    h = hashlib.sha256()
    for f in ("qblk_gemv.hip", "qblk_device.h"):
        with open(os.path.join(ROOT, "bit_block_quant_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Timer:
    """Capture `launch(i % n)` for i in range(n * rot) into a HIP graph (rot
    passes over the n rotating inputs); time replays.  Short kernels take
    several passes per graph so that the boundary between two replays is not
    part of every few launches."""

    def __init__(self, torch, launch, n, rot=1):
        self.torch = torch
        self.n = n * rot
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(n):  # eager pass (also loads the kernels)
                launch(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g):
            for i in range(n * rot):
                launch(i % n)
        torch.cuda.synchronize()

    def run(self, reps, warmup=1):
        t = self.torch
        for _ in range(warmup):
            self.g.replay()
        t.cuda.synchronize()
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            self.g.replay()
        b.record()
        t.cuda.synchronize()
        return a.elapsed_time(b) / (reps * self.n)  # ms per launch


def time_region(torch, fn):
    """ms for fn() on the current stream, HIP events, synchronized both sides."""
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b)


def hbm_reference(torch, dev, nbytes, C):
    """What torch's own copy kernel reaches on this GPU, beside the nominal
    8 TB/s: over the headline's byte count (C rotating buffers, so reads come
    from HBM) and over 1 GiB; bytes = read + write."""
    out = {}

    def rec(name, ms, nb):
        gbs = nb / (ms * 1e-3) / 1e9
        out[name] = {"us": round(ms * 1e3, 2), "GBps": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}
        log(f"  reference {name}: {ms * 1e3:.2f} us, {gbs:.0f} GB/s")

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
        traffic_run(torch, q, WL, dev)
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

    # exactly `steps` launches: a graph of G = whole passes over the C copies
    # (up to 2000 launches) replayed steps // G times, then a graph of the
    # remaining steps % G.  One graph per 24 launches instead measures the
    # replay boundary as well (7.34-7.46 against 7.22 us per launch).
    launch = lambda i: q.gemv(copies[i % C], q.SB4, M, K, xd, out=yd)  # noqa: E731
    G = C * max(1, min(args.steps, 2000) // C)
    full, rem = divmod(args.steps, G)
    g_full = Timer(torch, launch, C, G // C)
    g_rem = Timer(torch, launch, rem) if rem else None
    for i in range(args.warmup):  # untimed warmup launches
        launch(i)

    def region():
        for _ in range(full):
            g_full.g.replay()
        if g_rem is not None:
            g_rem.g.replay()

    steps = args.steps
    ms = time_region(torch, region) / steps
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
            "timing": "HIP graph of back-to-back launches, HIP events",
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


def traffic_run(torch, q, WL, dev):
    """A known-size streaming kernel (fp32 multiply: reads and writes
    CALIB_BYTES once each), then 8 GEMV launches on distinct copies of the
    headline blocks."""
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()
    del src, dst
    w, x = WL.sb4_decode("up")
    M, K = w.shape
    b0 = q.quantize(torch.from_numpy(w).to(dev), q.SB4)
    C = n_copies(b0.numel())
    cps = [b0] + [b0.clone() for _ in range(C - 1)]
    xd = torch.from_numpy(x).to(dev)
    y = torch.empty(M, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    for i in range(8):
        q.gemv(cps[(i + 1) % C], q.SB4, M, K, xd, out=y)
    torch.cuda.synchronize()
    log("traffic run done")


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
        hbm_row(name, ms, b0.numel() + x.numel() * x.element_size() + 4 * m, m=m, k=k)

    w, x = WL.sb4_decode("down")
    gemv_row("gemv_sb4_4096x11008_f16", q.SB4, torch.from_numpy(w).to(dev), torch.from_numpy(x).to(dev))
    w, x = WL.q4_0_decode()
    gemv_row("gemv_q4_0_4096x4096_f16", q.Q4_0, torch.from_numpy(w).to(dev), torch.from_numpy(x).to(dev))
    w, x = WL.q4_0_small()
    gemv_row("gemv_q4_0_256x4096_f32", q.Q4_0, torch.from_numpy(w).to(dev), torch.from_numpy(x).to(dev))
    w, x = WL.sb4_decode("up")
    gemv_row("gemv_q4k_11008x4096_f16", q.Q4_K, torch.from_numpy(w).to(dev), torch.from_numpy(x).to(dev))

    # quantizers
    def quant_row(name, fmt, w):
        # rotating input copies (past the last-level cache), one graph of C launches
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
    t = Timer(torch, lambda i: q.quantize(mats[i], q.SB4_AFFINE, out=outs[i]), n)
    ms = t.run(2) * n
    src = sum(m.numel() * 2 for m in mats)
    dst = sum(o.numel() for o in outs)
    hbm_row("quantize_sb4a_stack_32x7_f16", ms, src + dst,
            weights=sum(m.numel() for m in mats), weights_per_s=round(sum(m.numel() for m in mats) / (ms * 1e-3), 1))
    del mats
    ys = [torch.empty(WL.STACK_PROJ[i % 7][1], dtype=torch.float32, device=dev) for i in range(n)]

    def stack_gemv(i):
        _, r, k = WL.STACK_PROJ[i % 7]
        q.gemv(outs[i], q.SB4_AFFINE, r, k, xs[i], out=ys[i])

    t = Timer(torch, stack_gemv, n)
    ms = t.run(3) * n
    nb = dst + sum(xx.numel() * 2 for xx in xs) + sum(yy.numel() * 4 for yy in ys)
    hbm_row("gemv_sb4a_stack_32x7_f16", ms, nb, tokens_per_s_equivalent=round(1.0 / (ms * 1e-3), 1))
    del outs, xs, ys

    # prefill GEMM
    for shape in ("up", "down"):
        w, _ = WL.sb4_prefill(shape, 16)
        m, k = w.shape
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
                              frac_mfma_bf16=round(tf / BF16_PEAK_TFLOPS, 4))
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
    t = Timer(torch, lambda i: q.quantize_act_i8(xd, out=xq, scale=xs), 50)  # 50 launches per graph
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
def cpu_baseline(np, WL, w, x, algo_bytes, budget_s):
    """The oracle GEMV on the host: first on one thread, then on every host
    core (row chunks on a thread pool; the C oracle runs with the GIL
    released).  `value` is the all-cores rate; each leg gets half the budget."""
    import oracle as O
    from concurrent.futures import ThreadPoolExecutor

    m, k = w.shape
    blocks = O.quantize_sb4(w)  # the oracle quantizes its own input (untimed)
    xd = x.astype(np.float64)
    threads = max(1, min(len(os.sched_getaffinity(0)), 16))
    chunks = [np.arange(r0, min(m, r0 + (m + threads - 1) // threads), dtype=np.int64)
              for r0 in range(0, m, (m + threads - 1) // threads)]

    def timed(fn, budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget or reps >= 1000:
                return reps, el

    r1, e1 = timed(lambda: O.gemv(O.SB4, blocks, m, k, xd), budget_s / 2)
    with ThreadPoolExecutor(threads) as pool:
        def all_cores():
            list(pool.map(lambda rows: O.gemv(O.SB4, blocks, m, k, xd, rows=rows), chunks))
        rt, et = timed(all_cores, budget_s / 2)
    per1, pert = e1 / r1, et / rt
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), cpu)
    except OSError:
        pass
    return {
        "value": round(algo_bytes / pert / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"full {m}x{k} super-block GEMVs (C oracle: per-row fp32 dequant, fp64 sums); "
                  f"{rt} on {threads} threads in {et:.1f} s ({pert * 1e3:.1f} ms each), "
                  f"{r1} on 1 thread in {e1:.1f} s ({per1 * 1e3:.1f} ms each)",
        "single_thread": {"value": round(algo_bytes / per1 / 1e9, 3), "unit": "GB/s", "cores": 1},
        "host_cpu": cpu,
    }


if __name__ == "__main__":
    main()
