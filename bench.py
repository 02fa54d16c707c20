"""Benchmark of the SP-region forward + backward on one shard, one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

A step is one pass of the whole path over one shard: sp_region_fwd then
sp_region_bwd (its main kernel and the dgamma finish).  Inputs are seeded
synthetic tensors already resident in HBM.  Steps rotate over enough disjoint
buffer sets that one pass over them moves more than 1.5 GB, well beyond the
256 MB Infinity Cache, so every step reads HBM.

Timed region: K steps launched by replaying a captured HIP graph (so host
launch cost does not throttle the GPU), bracketed by synchronize on both sides
and timed by the host clock.  value = algorithmic bytes of fwd + bwd per step /
time per step.  A second pass replays forward-only and backward-only graphs
over all buffer sets between HIP event pairs recorded on the kernels' stream:
the elapsed time divided by the launches gives the per-launch durations behind
"roofline" (forward = the dominant kernel).  A 1 GiB device copy on the same
stream is timed as an achievable-bandwidth reference.

cpu_baseline: the CPU oracle, single-threaded, on a bounded sample of the same
shard's rows (about 10 s of work), with a parity check of those rows against
the GPU's outputs.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

DEFAULT_WORKLOAD = "layernorm_T8_S4096_B1_H4096"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
ROTATE_BYTES = 1.5e9
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--shard", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def source_digest():
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "transformer_sequence_activation_amd", "csrc", "sp_region.hip"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload):
    """HBM bytes per launch from a committed rocprofv3 FETCH/WRITE summary, if it
    was taken on the current kernel source."""
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest():
        return None
    return rec


class SetBuffers:
    """One disjoint set of inputs and outputs for one step."""

    def __init__(self, sp, w, j, src):
        import torch
        dev = "cuda"
        act = w.torch_dtype
        R, H = w.R, w.H
        self.P = [p.clone() for p in src["P"]]
        self.res = src["res"].clone()
        self.dY = src["dY"].clone()
        self.gamma = src["gamma"].clone()
        self.beta = None if src["beta"] is None else src["beta"].clone()
        ln = w.norm == "ln"
        self.h = torch.empty((R, H), dtype=act, device=dev)
        self.y = torch.empty((R, H), dtype=act, device=dev)
        self.mask = torch.empty((R, H), dtype=torch.uint8, device=dev)
        self.mean = torch.empty(R, device=dev) if ln else None
        self.rstd = torch.empty(R, device=dev)
        self.dres = torch.empty((R, H), dtype=act, device=dev)
        self.dP = torch.empty((R, H), dtype=act, device=dev)
        self.dgamma = torch.empty(H, device=dev)
        self.dbeta = torch.empty(H, device=dev) if ln else None
        d = sp.make_desc(w.S, w.B, w.H, w.T, j, w.dtype, w.norm, w.eps, w.p, w.seed)
        self.desc = d
        self.ws_bytes = max(16, sp.sp_region_bwd_workspace_size(d))
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)

    def prepare(self, sp, stream):
        self.fwd = sp.prepare_fwd(self.desc, self.P, self.res, self.gamma, self.beta, self.h, self.y,
                                  self.mask, self.mean, self.rstd, stream=stream)
        self.bwd = sp.prepare_bwd(self.desc, self.dY, self.h, self.mask, self.mean, self.rstd,
                                  self.gamma, None, self.dres, self.dP, self.dgamma, self.dbeta,
                                  self.ws, self.ws_bytes, stream=stream)


def cpu_baseline(sp, w, j, src, outs, seconds):
    """The oracle (plain C, one thread) on the first n rows of the shard."""
    import numpy as np
    import torch

    import oracle
    from transformer_sequence_activation_amd import workloads as W

    def u16(t):
        t = t.contiguous().cpu()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    od = oracle.make_desc(w.S, w.B, w.H, w.T, j, oracle.BF16 if w.dtype == "bf16" else oracle.F32,
                          oracle.LAYERNORM if w.norm == "ln" else oracle.RMSNORM, w.eps, w.p, w.seed)
    gam = src["gamma"].double().cpu().numpy()
    bet = None if src["beta"] is None else src["beta"].double().cpu().numpy()

    def run(n):
        P = [u16(W.shard(p, w, j)[:n]) for p in src["P"]]  # full partials: slice shard j
        res = u16(src["res"][:n])                           # already the shard
        dY = u16(src["dY"][:n])
        t0 = time.perf_counter()
        o = oracle.fwd(od, P, res, gam, bet, row0=0, nrows=n)
        ob = oracle.bwd(od, dY, o["h"], o["mask"],
                        None if o["mean"] is None else o["mean"].astype(np.float32).astype(np.float64),
                        o["rstd"].astype(np.float32).astype(np.float64), gam, row0=0, nrows=n)
        return time.perf_counter() - t0, o, ob

    probe = max(1, min(w.R, 4))
    t_probe, _, _ = run(probe)
    n = int(max(1, min(w.R, probe * seconds / max(t_probe, 1e-6))))
    t, o, ob = run(n)
    reps = 1
    while t * (reps + 1) / reps < seconds and reps < 1000:  # whole shard is quick: repeat it
        dt, _, _ = run(n)
        t += dt
        reps += 1
    t /= reps
    # algorithmic bytes of the sample (per-row share of the shard's bytes, plus the [H] vectors)
    fwd_b, bwd_b = sp.sp_region_traffic_bytes(sp.make_desc(w.S, w.B, w.H, w.T, j, w.dtype, w.norm))
    per_row = (fwd_b + bwd_b) / w.R
    sample_bytes = per_row * n
    # parity of the sample against the GPU's first set
    mask_ok = bool(np.array_equal(outs.mask[:n].cpu().numpy(), o["mask"]))
    h_ok = bool(np.array_equal(u16(outs.h[:n]), o["h"]))
    bf = oracle.bf16_to_f32 if w.dtype == "bf16" else (lambda a: a)

    def within(g, r, rtol):
        g = np.asarray(g, np.float64)
        r = np.asarray(r, np.float64)
        rms = math.sqrt(float(np.mean(r ** 2)))
        return bool(np.all(np.abs(g - r) <= rtol * np.abs(r) + rtol * rms))

    rt = 1e-2 if w.dtype == "bf16" else 1e-5
    y_ok = within(bf(u16(outs.y[:n])), bf(o["y"]), rt)
    dres_ok = within(bf(u16(outs.dres[:n])), bf(ob["d_res"]), rt)
    dp_ok = within(bf(u16(outs.dP[:n])), bf(ob["dP"]), rt)
    rstd_ok = within(outs.rstd[:n].cpu().numpy(), o["rstd"], 1e-5)
    parity = all([mask_ok, h_ok, y_ok, dres_ok, dp_ok, rstd_ok])
    return {
        "value": round(sample_bytes / t / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"forward + backward of rows 0..{n - 1} of shard {j} ({n} of {w.R} token rows, "
                  f"{sample_bytes / 1e6:.1f} MB algorithmic), {reps} run(s), {t:.3f} s each",
        "tokens_per_s": round(n / t, 2),
        "cpu": _cpu_model(),
        "parity_vs_gpu_sample": "pass" if parity else "FAIL",
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported by this build "
              "(the path has no collectives; see the sharding note in the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import transformer_sequence_activation_amd as sp
    from transformer_sequence_activation_amd import workloads as W

    sp.load()
    w = W.WORKLOADS[args.workload]
    j = w.shards[0] if args.shard is None else args.shard
    torch.cuda.set_device(0)
    src = {
        "P": [W.partial(w, t, "cuda") for t in range(w.T)],
        "res": W.shard(W.residual(w, "cuda"), w, j).clone(),
        "dY": W.shard(W.grad_y(w, "cuda"), w, j).clone(),
        "gamma": W.gamma(w, "cuda"),
        "beta": W.beta(w, "cuda"),
    }
    d0 = sp.make_desc(w.S, w.B, w.H, w.T, j, w.dtype, w.norm, w.eps, w.p, w.seed)
    fwd_bytes, bwd_bytes = sp.sp_region_traffic_bytes(d0)
    step_bytes = fwd_bytes + bwd_bytes
    n_sets = max(2, math.ceil(ROTATE_BYTES / step_bytes))
    n_sets = min(n_sets, args.steps) if args.steps >= 2 else n_sets
    stream = torch.cuda.Stream()
    sets = [SetBuffers(sp, w, j, src) for _ in range(n_sets)]
    for s in sets:
        s.prepare(sp, stream.cuda_stream)

    def step(s):
        s.fwd()
        s.bwd()

    # eager run on every set (also the warm start of the allocator and code objects)
    with torch.cuda.stream(stream):
        for s in sets:
            step(s)
    torch.cuda.synchronize()

    # graphs: one pass over all sets, one for the remainder of K, and forward-only
    # / backward-only passes for the per-launch durations
    K, Wm = args.steps, args.warmup
    reps, rem = divmod(K, n_sets)

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn()
        return g

    g_all = capture(lambda: [step(s) for s in sets])
    g_rem = capture(lambda: [step(s) for s in sets[:rem]]) if rem else None
    g_fwd = capture(lambda: [s.fwd() for s in sets])
    g_bwd = capture(lambda: [s.bwd() for s in sets])
    torch.cuda.synchronize()
    # graph replays must reproduce the eager results bit for bit
    keys = ("h", "y", "mask", "rstd", "dres", "dP", "dgamma")
    ref = {k: getattr(sets[0], k).clone() for k in keys}
    graph_ok = True
    for _ in range(2):
        for s in sets:
            for k in ("h", "y", "dres", "dP"):
                getattr(s, k).zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g_all.replay()
        torch.cuda.synchronize()
        graph_ok = graph_ok and all(torch.equal(ref[k], getattr(sets[0], k)) for k in keys)

    def replay(g, times=1):
        with torch.cuda.stream(stream):
            for _ in range(times):
                g.replay()

    # warmup
    replay(g_all, max(1, math.ceil(Wm / n_sets)))
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps ----
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        ev0.record(stream)
        for _ in range(reps):
            g_all.replay()
        if g_rem is not None:
            g_rem.replay()
        ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = wall_ms / K

    # ---- per-launch durations: HIP events on the kernels' stream around
    # back-to-back forward launches (one per buffer set), then backward launches
    ev_reps = max(4, min(50, math.ceil(2000 / n_sets)))
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(ev_reps)]
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for m in marks:
            m[0].record(stream)
            g_fwd.replay()
            m[1].record(stream)
            g_bwd.replay()
            m[2].record(stream)
    torch.cuda.synchronize()
    fwd_us = sorted(m[0].elapsed_time(m[1]) * 1e3 / n_sets for m in marks)
    bwd_us = sorted(m[1].elapsed_time(m[2]) * 1e3 / n_sets for m in marks)
    fwd_avg = sum(fwd_us) / ev_reps
    bwd_avg = sum(bwd_us) / ev_reps

    # ---- reference: a plain device-to-device copy of 1 GiB, same stream ----
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    with torch.cuda.stream(stream):
        b.copy_(a)
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(10):
            b.copy_(a)
        c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * a.numel() * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del a, b

    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = fwd_bytes / (fwd_avg * 1e-6) / 1e9
    traffic = load_traffic(w.name)
    line = {
        "metric": "achieved HBM GB/s (and % of peak) for SP-region fused fwd+bwd on one shard",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "S": w.S, "B": w.B, "H": w.H, "shard": j,
                   "norm": w.norm, "p": w.p, "eps": w.eps, "parallelism": "one shard, 1 GPU"},
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "tokens_per_s": round(w.R / (ms_per_step * 1e-3), 1),
        "bytes_per_step": step_bytes,
        "fwd_bytes": fwd_bytes,
        "bwd_bytes": bwd_bytes,
        "buffer_sets": n_sets,
        "timing": {"method": "hip graph replay, host clock", "gpu_event_ms_per_step": round(gpu_ms / K, 6),
                   "fwd_us_avg": round(fwd_avg, 3), "fwd_us_median": round(fwd_us[ev_reps // 2], 3),
                   "bwd_us_avg": round(bwd_avg, 3), "bwd_us_median": round(bwd_us[ev_reps // 2], 3),
                   "event_launches_each": ev_reps * n_sets, "graph_replay_matches_eager": graph_ok},
        "copy_reference_GBs": round(copy_gbs, 1),
        "roofline": {
            "kernel": "sp_fwd_kernel",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": None if traffic is None else traffic["fwd_bytes_per_launch"],
        },
        "cpu_baseline": None,
    }
    if traffic is not None:
        line["roofline"]["traffic_detail"] = traffic
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(sp, w, j, src, sets[0], args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
