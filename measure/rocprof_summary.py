"""Summarise a rocprofv3 results database: per-kernel durations (from the
kernel trace, and rocprofv3's own --stats summary) and, when the run collected
them, the FETCH_SIZE / WRITE_SIZE hardware counters.

    python -m measure.rocprof_summary RESULTS.db [...]
        [--copy-bytes N] [--filter SUBSTRING]

FETCH_SIZE and WRITE_SIZE are reported by the profiler in KiB per dispatch.
With --copy-bytes N, the largest device-copy dispatch in the same database
(rocclr's copyBuffer; bench.py --profile-pass makes it a copy of N bytes)
calibrates them: bytes = counter * N / counter(copy).  On gfx950, FETCH_SIZE of
a copy reads half of the bytes copied, WRITE_SIZE all of them.

--traffic-json PATH writes the per-launch bytes of the forward and backward
kernels, with the digest of the kernel source they were taken on.
"""
import argparse
import re
import sqlite3
from collections import defaultdict


def short_name(name):
    n = re.sub(r"\(anonymous namespace\)::", "", name)
    n = re.sub(r"^void ", "", n)
    return re.sub(r"\((?!.*<).*$", "", n)[:90]


def kernel_stats(con, filt=None):
    rows = con.execute("select name, duration from kernels").fetchall()
    acc = defaultdict(list)
    for name, dur in rows:
        if filt and filt not in name:
            continue
        acc[short_name(name)].append(dur)
    out = []
    for k, v in acc.items():
        v.sort()
        out.append((k, len(v), sum(v) / len(v) / 1e3, v[0] / 1e3, v[len(v) // 2] / 1e3, v[-1] / 1e3))
    return sorted(out, key=lambda r: -r[1] * r[2])


def rocprof_stats(con, filt=None):
    """rocprofv3's own --stats summary, kept in the results database as the
    top_kernels view: (name, calls, total_us, average_us, percent)."""
    tables = {r[0] for r in con.execute("select name from sqlite_master where type in ('table','view')")}
    if "top_kernels" not in tables:
        return []
    rows = con.execute("select name, total_calls, total_duration, average, percentage from top_kernels")
    return [(short_name(n), int(c), float(t), float(av), float(pc)) for n, c, t, av, pc in rows
            if not filt or filt in n]


def counters(con):
    """{kernel short name: {counter: [values per dispatch]}} if counters were collected."""
    tables = {r[0] for r in con.execute("select name from sqlite_master where type in ('table','view')")}
    if "counters_collection" not in tables:
        return {}
    cols = [r[1] for r in con.execute("pragma table_info(counters_collection)")]
    name_col = "kernel_name" if "kernel_name" in cols else "name"
    q = f"select {name_col}, counter_name, value, dispatch_id from counters_collection"
    per = defaultdict(lambda: defaultdict(lambda: defaultdict(float)))
    for kname, cname, val, disp in con.execute(q):
        per[short_name(kname)][cname][disp] += val
    return {k: {c: sorted(d.values()) for c, d in v.items()} for k, v in per.items()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("db", nargs="+")
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--filter", default=None)
    ap.add_argument("--traffic-json", default=None)
    ap.add_argument("--source-digest", default=None)
    a = ap.parse_args()
    traffic = {}
    for db in a.db:
        con = sqlite3.connect(db)
        print(f"# {db}")
        print(f"{'kernel':90s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'med_us':>9s} {'max_us':>9s}")
        for k, n, avg, mn, med, mx in kernel_stats(con, a.filter):
            print(f"{k:90s} {n:6d} {avg:9.3f} {mn:9.3f} {med:9.3f} {mx:9.3f}")
        st = rocprof_stats(con, a.filter)
        if st:
            print("\nrocprofv3 --stats (top_kernels view)")
            print(f"{'kernel':90s} {'calls':>6s} {'total_us':>11s} {'avg_us':>9s} {'percent':>8s}")
            for k, n, tot, avg, pc in st:
                print(f"{k:90s} {n:6d} {tot:11.1f} {avg:9.3f} {pc:8.2f}")
        cnt = counters(con)
        if cnt:
            scale = {}
            if a.copy_bytes:
                copy = [k for k in cnt if "copyBuffer" in k]
                for c in ("FETCH_SIZE", "WRITE_SIZE"):
                    vals = [v for k in copy for v in cnt[k].get(c, [])]
                    if vals and max(vals) > 0:
                        scale[c] = a.copy_bytes / max(vals)
            print()
            print(f"{'kernel':90s} {'counter':>11s} {'n':>4s} {'median':>12s} {'bytes(scaled)':>14s}")
            for k, cs in sorted(cnt.items()):
                if a.filter and a.filter not in k and "copyBuffer" not in k:
                    continue
                for c, vals in sorted(cs.items()):
                    med = vals[len(vals) // 2]
                    sb = f"{med * scale[c]:14.0f}" if scale.get(c) else f"{'':14s}"
                    print(f"{k:90s} {c:>11s} {len(vals):4d} {med:12.1f} {sb}")
            if scale:
                print("\ncalibration (bytes per counter unit from the copy kernel):",
                      {c: round(v, 3) for c, v in scale.items() if v})
                for k, cs in cnt.items():
                    for tag in ("sp_fwd_kernel", "sp_bwd_kernel", "sp_dgamma_finish_kernel"):
                        if k.startswith(tag):
                            for c, vals in cs.items():
                                if scale.get(c):
                                    traffic[f"{tag}:{c}"] = vals[len(vals) // 2] * scale[c]
    if a.traffic_json and traffic:
        import json
        rec = {
            "source_digest": a.source_digest,
            "fwd_bytes_per_launch": round(traffic.get("sp_fwd_kernel:FETCH_SIZE", 0)
                                          + traffic.get("sp_fwd_kernel:WRITE_SIZE", 0)),
            "fwd_fetch_bytes": round(traffic.get("sp_fwd_kernel:FETCH_SIZE", 0)),
            "fwd_write_bytes": round(traffic.get("sp_fwd_kernel:WRITE_SIZE", 0)),
            "bwd_main_fetch_bytes": round(traffic.get("sp_bwd_kernel:FETCH_SIZE", 0)),
            "bwd_main_write_bytes": round(traffic.get("sp_bwd_kernel:WRITE_SIZE", 0)),
            "bwd_finish_fetch_bytes": round(traffic.get("sp_dgamma_finish_kernel:FETCH_SIZE", 0)),
            "bwd_finish_write_bytes": round(traffic.get("sp_dgamma_finish_kernel:WRITE_SIZE", 0)),
            "calibration": "FETCH_SIZE / WRITE_SIZE medians per dispatch, scaled by the largest "
                           "copyBuffer dispatch (the 256 MiB reference copy)",
        }
        with open(a.traffic_json, "w") as f:
            json.dump(rec, f, indent=1)
        print(f"wrote {a.traffic_json}")


if __name__ == "__main__":
    main()
