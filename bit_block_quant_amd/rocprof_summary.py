"""Summaries of rocprofv3 output directories (the SQLite results it writes).

    python -m bit_block_quant_amd.rocprof_summary trace DIR
        per-kernel dispatch count and duration statistics (--kernel-trace)
    python -m bit_block_quant_amd.rocprof_summary pmc DIR
        per-kernel mean of every collected counter (--pmc)
    python -m bit_block_quant_amd.rocprof_summary traffic FETCH_DIR WRITE_DIR KERNEL_SUBSTR
        HBM bytes per launch of one kernel from a FETCH_SIZE run and a
        WRITE_SIZE run, each scaled by the same counter's reading for the
        256 MiB fp32 multiply kernel (reads and writes 256 MiB) that
        `bench.py --mode traffic` runs first; prints JSON.
"""
import collections
import glob
import json
import os
import sqlite3
import statistics
import sys

CALIB_BYTES = 256 << 20
CALIB_KERNEL = "MulFunctor"  # torch's fp32 multiply kernel


def _db(d):
    dbs = sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))
    if not dbs:
        raise SystemExit(f"no rocprofv3 database under {d}")
    return sqlite3.connect(dbs[0])


def _pct(ds, p):
    s = sorted(ds)
    return s[min(len(s) - 1, int(round(p / 100.0 * (len(s) - 1))))]


def trace(d):
    c = _db(d)
    rows = c.execute("select name, start, end from kernels order by start").fetchall()
    by = collections.defaultdict(list)
    for n, s, e in rows:
        by[n].append((e - s) / 1000.0)
    out = []
    for n, ds in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        out.append(dict(kernel=n, calls=len(ds), total_us=round(sum(ds), 3), avg_us=round(statistics.mean(ds), 3),
                        median_us=round(statistics.median(ds), 3), p10_us=round(_pct(ds, 10), 3),
                        p90_us=round(_pct(ds, 90), 3), min_us=round(min(ds), 3),
                        max_us=round(max(ds), 3)))
    return out


def pmc(d):
    c = _db(d)
    rows = c.execute("select kernel_name, dispatch_id, counter_name, sum(value) from counters_collection "
                     "group by dispatch_id, counter_name").fetchall()
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for k, _, cn, v in rows:
        agg[k][cn].append(v)
    return {k: {cn: dict(n=len(vs), mean=statistics.mean(vs)) for cn, vs in cs.items()} for k, cs in agg.items()}


def _counter(d, counter, substr):
    res = pmc(d)
    calib = [v[counter]["mean"] for k, v in res.items() if CALIB_KERNEL in k and counter in v]
    kern = [v[counter] for k, v in res.items() if substr in k and counter in v]
    if not calib or not kern:
        raise SystemExit(f"{counter}: calibration copy or kernel '{substr}' not found in {d}")
    return max(calib), kern[0]["mean"], kern[0]["n"]


def traffic(fetch_dir, write_dir, substr):
    f_cal, f_k, n_f = _counter(fetch_dir, "FETCH_SIZE", substr)
    w_cal, w_k, n_w = _counter(write_dir, "WRITE_SIZE", substr)
    # counters are in KiB; the copy moved CALIB_BYTES each way
    f_factor = CALIB_BYTES / (f_cal * 1024.0)
    w_factor = CALIB_BYTES / (w_cal * 1024.0)
    fetch = f_k * 1024.0 * f_factor
    write = w_k * 1024.0 * w_factor
    return dict(kernel_substr=substr, fetch_kib_raw=f_k, write_kib_raw=w_k, calib_fetch_kib=f_cal,
                calib_write_kib=w_cal, fetch_factor=round(f_factor, 4), write_factor=round(w_factor, 4),
                fetch_bytes=round(fetch), write_bytes=round(write), bytes_per_launch=round(fetch + write),
                dispatches=[n_f, n_w])


if __name__ == "__main__":
    cmd = sys.argv[1] if len(sys.argv) > 1 else ""
    if cmd == "trace":
        for r in trace(sys.argv[2]):
            print(f"{r['calls']:6d}  avg {r['avg_us']:10.3f} us  med {r['median_us']:10.3f}  "
                  f"p10 {r['p10_us']:10.3f}  p90 {r['p90_us']:10.3f}  min {r['min_us']:10.3f}  max {r['max_us']:10.3f}  total {r['total_us']:12.1f}  {r['kernel'][:110]}")
    elif cmd == "pmc":
        for k, cs in pmc(sys.argv[2]).items():
            print(k[:110])
            for cn, v in sorted(cs.items()):
                print(f"    {cn:28s} n={v['n']:5d} mean={v['mean']:.6g}")
    elif cmd == "traffic":
        print(json.dumps(traffic(sys.argv[2], sys.argv[3], sys.argv[4]), indent=1))
    else:
        print(__doc__)
        sys.exit(2)
