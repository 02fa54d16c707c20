"""Benchmark of the SP-region forward + backward, one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

A step is one pass of the whole path over one batch: sp_region_fwd then
sp_region_bwd (its main kernel and the dgamma finish) on one shard -- or, for
the long-sequence workload, on all of its shards one after another.  Inputs are
seeded synthetic tensors already resident in HBM.  Steps rotate over enough
disjoint buffer sets that one pass over them moves more than 1.5 GB, well beyond
the 256 MB Infinity Cache, so every step reads HBM.

Timed region: exactly K steps, launched directly on one stream (measured at
least as fast as replaying a captured HIP graph of the same launches: the host
keeps ahead of the GPU), bracketed by synchronize on both sides and timed by the
host clock; HIP events on the stream time the same K steps as well.  The
launches run the forwards of all buffer sets, then their backwards, so a
batch's backward does not find its forward's outputs in the caches.  value =
algorithmic bytes of fwd + bwd per step / time per step.  A second pass
launches the forwards of all buffer sets, then their backwards, between HIP
event pairs recorded on the kernels' stream: elapsed time / launches gives the
per-launch durations behind "roofline" (the forward is the dominant kernel).
A graph captured from the same launches is replayed twice and must reproduce
the eager outputs bit for bit.  A 1 GiB device copy on the same stream is timed as an
achievable-bandwidth reference.  The other workloads are measured the same way
with fewer steps and reported under "workloads"; a step of those covers every
shard the workload lists (MiniMind: shards 0 and 1; long sequence: all 8).

cpu_baseline: the CPU oracle on a bounded sample of the headline shard, with a
parity check of that sample against the GPU's outputs: once on one thread
(about 10 s of work) and once split into row blocks over the host cores this
process may use, at most 16 (about 5 s); `value` and `cores` are the threaded
run's.  "warm" figures repeat one buffer set, which stays in the Infinity
Cache when a step's bytes fit there: cache-resident, not HBM.
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
# (workload, descriptor flags): the other workloads, and the headline and large-hidden shards
# with the mask regenerated in the backward instead of stored (SP_FLAG_RECOMPUTE_MASK)
SECONDARY = [("minimind_T2_S2048_B2_H768", 0), ("large_hidden_T8_S8192_B2_H8192", 0),
             ("long_seq_T8_S32768_B1_H8192", 0), (DEFAULT_WORKLOAD, 1),
             ("large_hidden_T8_S8192_B2_H8192", 1)]
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
CPU_SHARE = 16  # host cores one GPU's work may use on a shared host
ROTATE_BYTES = 1.5e9
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--profile-pass", action="store_true",
                    help="no timing: run a few eager forward/backward launches on cold buffer sets "
                         "and a 256 MiB device copy (the reference for hardware byte counters), "
                         "for use under rocprofv3")
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


class ShardBuffers:
    """Per-shard inputs and outputs of one buffer set."""

    def __init__(self, sp, w, j, src, P, flags=0):
        import torch
        dev, act, R, H = "cuda", w.torch_dtype, w.R, w.H
        ln = w.norm == "ln"
        self.j = j
        self.P = P
        self.res = src["res"][j].clone()
        self.dY = src["dY"][j].clone()
        self.gamma = src["gamma"]
        self.beta = src["beta"]
        self.h = torch.empty((R, H), dtype=act, device=dev)
        self.y = torch.empty((R, H), dtype=act, device=dev)
        regen = flags & sp.SP_FLAG_RECOMPUTE_MASK
        self.mask = None if regen else torch.empty((R, H), dtype=torch.uint8, device=dev)
        self.mean = torch.empty(R, device=dev) if ln else None
        self.rstd = torch.empty(R, device=dev)
        self.dres = torch.empty((R, H), dtype=act, device=dev)
        self.dP = torch.empty((R, H), dtype=act, device=dev)
        self.dgamma = torch.empty(H, device=dev)
        self.dbeta = torch.empty(H, device=dev) if ln else None
        self.desc = sp.make_desc(w.S, w.B, w.H, w.T, j, w.dtype, w.norm, w.eps, w.p, w.seed, flags)
        self.ws_bytes = max(16, sp.sp_region_bwd_workspace_size(self.desc))
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=dev)  # zero-filled once

    def prepare(self, sp, stream):
        self.fwd = sp.prepare_fwd(self.desc, self.P, self.res, self.gamma, self.beta, self.h, self.y,
                                  self.mask, self.mean, self.rstd, stream=stream)
        self.bwd = sp.prepare_bwd(self.desc, self.dY, self.h, self.mask, self.mean, self.rstd,
                                  self.gamma, None, self.dres, self.dP, self.dgamma, self.dbeta,
                                  self.ws, self.ws_bytes, stream=stream)


class BufferSet:
    """One disjoint set: its own copy of the full partial buffers and the shards' tensors."""

    def __init__(self, sp, w, shards, src, flags=0):
        self.P = [p.clone() for p in src["P"]]
        self.shards = [ShardBuffers(sp, w, j, src, self.P, flags) for j in shards]

    def prepare(self, sp, stream):
        for s in self.shards:
            s.prepare(sp, stream)

    def step(self):
        for s in self.shards:
            s.fwd()
            s.bwd()


def make_source(w, shards):
    """Seeded inputs on the GPU: full partials, per-shard residual / dY slices."""
    from transformer_sequence_activation_amd import workloads as W
    res = W.residual(w, "cuda")
    dY = W.grad_y(w, "cuda")
    src = {
        "P": [W.partial(w, t, "cuda") for t in range(w.T)],
        "res": {j: W.shard(res, w, j).clone() for j in shards},
        "dY": {j: W.shard(dY, w, j).clone() for j in shards},
        "gamma": W.gamma(w, "cuda"),
        "beta": W.beta(w, "cuda"),
    }
    del res, dY
    return src


def measure(sp, w, shards, K, Wm, stream, flags=0, paired=False):
    """Time K steps (graph replay, host clock) and per-launch durations (events).

    The timed graphs run the forwards of all buffer sets, then their backwards,
    so other sets' traffic (more than the 256 MB Infinity Cache) separates a
    batch's forward from its backward, as the rest of a model would: the
    backward cannot find h and the mask still cached.  paired=True runs each
    set's forward and backward back to back instead."""
    import torch

    src = make_source(w, shards)
    fwd_b = bwd_b = 0
    for j in shards:
        f, b = sp.sp_region_traffic_bytes(sp.make_desc(w.S, w.B, w.H, w.T, j, w.dtype, w.norm,
                                                       flags=flags))
        fwd_b += f
        bwd_b += b
    step_bytes = fwd_b + bwd_b
    n_sets = max(2, math.ceil(ROTATE_BYTES / step_bytes))
    n_sets = min(n_sets, max(2, K))
    sets = [BufferSet(sp, w, shards, src, flags) for _ in range(n_sets)]
    for s in sets:
        s.prepare(sp, stream.cuda_stream)
    torch.cuda.synchronize()  # the copies above ran on torch's current stream, not on `stream`
    with torch.cuda.stream(stream):
        for s in sets:
            s.step()
    torch.cuda.synchronize()

    reps, rem = divmod(K, n_sets)

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn()
        return g

    def steps(sel):
        def run():
            if paired:
                for s in sel:
                    s.step()
                return
            for s in sel:
                for sh in s.shards:
                    sh.fwd()
            for s in sel:
                for sh in s.shards:
                    sh.bwd()
        return run

    # a captured graph of the same launches must reproduce the eager results
    # bit for bit (the library enqueues kernels only)
    g_all = capture(steps(sets))
    torch.cuda.synchronize()

    first = sets[0].shards[0]
    keys = tuple(k for k in ("h", "y", "mask", "rstd", "dres", "dP", "dgamma")
                 if getattr(first, k) is not None)
    ref = {k: getattr(first, k).clone() for k in keys}
    graph_bad = set()
    for _ in range(2):
        for s in sets:
            for sh in s.shards:
                for k in ("h", "y", "dres", "dP", "dgamma"):
                    getattr(sh, k).zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g_all.replay()
        torch.cuda.synchronize()
        graph_bad |= {k for k in keys if not torch.equal(ref[k], getattr(first, k))}
    graph_ok = not graph_bad

    run_all, run_rem = steps(sets), steps(sets[:rem])
    with torch.cuda.stream(stream):
        for _ in range(max(1, math.ceil(Wm / n_sets))):
            run_all()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps, launched directly (measured at least
    # as fast as replaying the captured graph: the host launches keep ahead of
    # the GPU on these workloads) ----
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        ev0.record(stream)
        for _ in range(reps):
            run_all()
        if rem:
            run_rem()
        ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    gpu_ms_per_step = ev0.elapsed_time(ev1) / K

    # ---- per-launch durations: HIP events on the kernels' stream around
    # back-to-back forward launches (one per buffer set and shard), then backward
    launches = n_sets * len(shards)
    ev_reps = max(4, min(50, math.ceil(2000 / launches)))
    marks = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(ev_reps)]
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for m in marks:
            m[0].record(stream)
            for s in sets:
                for sh in s.shards:
                    sh.fwd()
            m[1].record(stream)
            for s in sets:
                for sh in s.shards:
                    sh.bwd()
            m[2].record(stream)
    torch.cuda.synchronize()
    fwd_us = sorted(m[0].elapsed_time(m[1]) * 1e3 / launches for m in marks)
    bwd_us = sorted(m[1].elapsed_time(m[2]) * 1e3 / launches for m in marks)

    # ---- warm: one buffer set over and over.  Where a step's bytes fit in the
    # 256 MB Infinity Cache this is cache-resident, not an HBM figure.
    n_warm = 32
    warm_reps = max(2, min(20, math.ceil(2000 / n_warm)))
    with torch.cuda.stream(stream):
        for _ in range(n_warm):
            sets[0].step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for _ in range(warm_reps * n_warm):
            sets[0].step()
    torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - t0) * 1e3 / (n_warm * warm_reps)
    out = {
        "workload": w.name, "shards": list(shards), "steps": K,
        "ms_per_step": ms_per_step, "gpu_event_ms_per_step": gpu_ms_per_step,
        "value_GBs": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "tokens_per_s": w.R * len(shards) / (ms_per_step * 1e-3),
        "bytes_per_step": step_bytes, "fwd_bytes": fwd_b // len(shards), "bwd_bytes": bwd_b // len(shards),
        "buffer_sets": n_sets,
        "fwd_us_avg": sum(fwd_us) / ev_reps, "fwd_us_median": fwd_us[ev_reps // 2],
        "bwd_us_avg": sum(bwd_us) / ev_reps, "bwd_us_median": bwd_us[ev_reps // 2],
        "event_launches_each": ev_reps * launches,
        "graph_replay_matches_eager": graph_ok,
        "graph_replay_mismatch": sorted(graph_bad),
        "warm_ms_per_step": warm_ms, "warm_GBs": step_bytes / (warm_ms * 1e-3) / 1e9,
        "warm_cache_resident": step_bytes < 256e6,
    }
    return out, src, sets


def roofline_entries(head, traffic):
    """Roofline of the forward (the dominant kernel) and of the backward (its
    main kernel plus the dgamma finish kernel where that schedule runs):
    algorithmic bytes per launch over the launch duration measured with HIP
    events on the kernels' stream; traffic = FETCH_SIZE + WRITE_SIZE per launch
    from the committed counter summary of the same kernel source, else null."""
    out = []
    for direction, nbytes, us in (("fwd", head["fwd_bytes"], head["fwd_us_avg"]),
                                  ("bwd", head["bwd_bytes"], head["bwd_us_avg"])):
        achieved = nbytes / (us * 1e-6) / 1e9
        t = None
        if traffic is not None:
            if direction == "fwd":
                t = traffic["fwd_bytes_per_launch"]
            else:
                t = (traffic["bwd_main_fetch_bytes"] + traffic["bwd_main_write_bytes"] +
                     traffic["bwd_finish_fetch_bytes"] + traffic["bwd_finish_write_bytes"])
        out.append({"kernel": "sp_fwd_kernel" if direction == "fwd" else
                    "sp_bwd_kernel (+ sp_dgamma_finish_kernel where it runs)",
                    "direction": direction, "bound": "hbm", "algorithmic_bytes": nbytes,
                    "launch_us": round(us, 3), "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": t,
                    "traffic_over_algorithmic": None if t is None else round(t / nbytes, 3)})
    return out


def copy_reference(stream):
    import torch
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
    return 2 * a.numel() * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9


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
        res = u16(src["res"][j][:n])
        dY = u16(src["dY"][j][:n])
        t0 = time.perf_counter()
        o = oracle.fwd(od, P, res, gam, bet, row0=0, nrows=n)
        ob = oracle.bwd(od, dY, o["h"], o["mask"],
                        None if o["mean"] is None else o["mean"].astype(np.float32).astype(np.float64),
                        o["rstd"].astype(np.float32).astype(np.float64), gam, row0=0, nrows=n)
        return time.perf_counter() - t0, o, ob

    probe = max(1, min(w.R, 4))
    t_probe, _, _ = run(probe)
    t_probe = max(t_probe, 1e-6)
    n = int(max(1, min(w.R, probe * seconds / max(t_probe, 1e-6))))
    t, o, ob = run(n)
    reps = 1
    while t * (reps + 1) / reps < seconds and reps < 1000:  # the whole shard is quick: repeat it
        dt, _, _ = run(n)
        t += dt
        reps += 1
    t /= reps
    fwd_b, bwd_b = sp.sp_region_traffic_bytes(sp.make_desc(w.S, w.B, w.H, w.T, j, w.dtype, w.norm))
    sample_bytes = (fwd_b + bwd_b) / w.R * n
    mask_ok = bool(np.array_equal(outs.mask[:n].cpu().numpy(), o["mask"]))
    h_ok = bool(np.array_equal(u16(outs.h[:n]), o["h"]))
    bf = oracle.bf16_to_f32 if w.dtype == "bf16" else (lambda a: a)

    def within(g, r, rtol):
        g = np.asarray(g, np.float64)
        r = np.asarray(r, np.float64)
        rms = math.sqrt(float(np.mean(r ** 2)))
        return bool(np.all(np.abs(g - r) <= rtol * np.abs(r) + rtol * rms))

    rt = 1e-2 if w.dtype == "bf16" else 1e-5
    parity = all([mask_ok, h_ok,
                  within(bf(u16(outs.y[:n])), bf(o["y"]), rt),
                  within(bf(u16(outs.dres[:n])), bf(ob["d_res"]), rt),
                  within(bf(u16(outs.dP[:n])), bf(ob["dP"]), rt),
                  within(outs.rstd[:n].cpu().numpy(), o["rstd"], 1e-5)])
    # the same oracle calls on disjoint row blocks from a thread pool (the C
    # oracle runs without the interpreter lock), on the host cores this process
    # may use, at most 16: one GPU's share of the host's cores, which the
    # affinity mask of a shared host may not reflect
    affinity = len(os.sched_getaffinity(0))
    threads = max(1, min(CPU_SHARE, affinity))
    nt = int(max(1, min(w.R, probe * seconds * threads / t_probe / 2)))
    blocks = [(r0, min(nt, r0 + max(1, math.ceil(nt / threads))))
              for r0 in range(0, nt, max(1, math.ceil(nt / threads)))]
    P_all = [u16(W.shard(p, w, j)[:nt]) for p in src["P"]]
    res_all, dY_all = u16(src["res"][j][:nt]), u16(src["dY"][j][:nt])

    def run_block(b):
        r0, r1 = b
        o = oracle.fwd(od, [p[r0:r1] for p in P_all], res_all[r0:r1], gam, bet, row0=r0, nrows=r1 - r0)
        oracle.bwd(od, dY_all[r0:r1], o["h"], o["mask"],
                   None if o["mean"] is None else o["mean"].astype(np.float32).astype(np.float64),
                   o["rstd"].astype(np.float32).astype(np.float64), gam, row0=r0, nrows=r1 - r0)

    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=threads) as ex:
        tt, treps = 0.0, 0
        while treps < 1 or (tt * (treps + 1) / treps < seconds / 2 and treps < 1000):
            t0 = time.perf_counter()
            list(ex.map(run_block, blocks))
            tt += time.perf_counter() - t0
            treps += 1
    tt /= treps
    threaded_bytes = (fwd_b + bwd_b) / w.R * nt
    return {
        "value": round(threaded_bytes / tt / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "cores_in_affinity_mask": affinity,
        "cores_note": f"threads = min({CPU_SHARE}, cores in the affinity mask): {CPU_SHARE} host cores are one "
                      "GPU's share of a shared host",
        "kind": "oracle",
        "single_thread_value": round(sample_bytes / t / 1e9, 4),
        "threaded_sample": f"rows 0..{nt - 1} of shard {j} in {len(blocks)} blocks on {threads} threads, "
                           f"{treps} run(s), {tt:.3f} s each",
        "sample": f"forward + backward of rows 0..{n - 1} of shard {j} ({n} of {w.R} token rows, "
                  f"{sample_bytes / 1e6:.1f} MB algorithmic), single thread: {reps} run(s), {t:.3f} s each",
        "tokens_per_s": round(nt / tt, 2),
        "single_thread_tokens_per_s": round(n / t, 2),
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


def profile_pass(sp, w, stream):
    """Eager launches for rocprofv3: a 256 MiB copy, then every set three times."""
    import torch
    shards = (w.shards[0],)
    src = make_source(w, shards)
    f, b = sp.sp_region_traffic_bytes(sp.make_desc(w.S, w.B, w.H, w.T, shards[0], w.dtype, w.norm))
    n_sets = max(2, math.ceil(ROTATE_BYTES / (f + b)))
    sets = [BufferSet(sp, w, shards, src) for _ in range(n_sets)]
    for s in sets:
        s.prepare(sp, stream.cuda_stream)
    a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    c = torch.empty_like(a)
    torch.cuda.synchronize()  # buffer copies ran on torch's current stream
    with torch.cuda.stream(stream):
        for _ in range(3):
            c.copy_(a)
        for _ in range(3):
            for s in sets:
                s.step()
    torch.cuda.synchronize()
    print(json.dumps({"profile_pass": w.name, "shard": shards[0], "buffer_sets": n_sets,
                      "copy_bytes": a.numel(), "fwd_bytes": f, "bwd_bytes": b}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the library runs one "
              "rank's shard on one GPU and has no collectives.", file=sys.stderr)
        sys.exit(2)

    import torch

    import transformer_sequence_activation_amd as sp
    from transformer_sequence_activation_amd import workloads as W

    import __graft_entry__
    __graft_entry__.build_if_missing()
    sp.load()
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    w = W.WORKLOADS[args.workload]
    if args.profile_pass:
        profile_pass(sp, w, stream)
        return

    j = w.shards[0]
    head, src, sets = measure(sp, w, (j,), args.steps, args.warmup, stream)
    copy_gbs = copy_reference(stream)
    traffic = load_traffic(w.name)
    kernels = roofline_entries(head, traffic)
    fwd_k = kernels[0]
    line = {
        "metric": "achieved HBM GB/s (and % of peak) for SP-region fused fwd+bwd on one shard",
        "value": round(head["value_GBs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "S": w.S, "B": w.B, "H": w.H, "shard": j,
                   "norm": w.norm, "p": w.p, "eps": w.eps, "parallelism": "one shard, 1 GPU"},
        "pct_of_peak": round(100 * head["value_GBs"] / PEAK_HBM_GBS, 2),
        "tokens_per_s": round(head["tokens_per_s"], 1),
        "bytes_per_step": head["bytes_per_step"],
        "fwd_bytes": head["fwd_bytes"],
        "bwd_bytes": head["bwd_bytes"],
        "buffer_sets": head["buffer_sets"],
        "timing": {"method": "direct launches on one stream, host clock",
                   "value_basis": "host clock around exactly K steps, synchronize on both sides "
                                  "(includes the latency of the first launch and of the final synchronize)",
                   "gpu_event_ms_per_step": round(head["gpu_event_ms_per_step"], 6),
                   "gpu_event_GBs": round(head["bytes_per_step"] / (head["gpu_event_ms_per_step"] * 1e-3) / 1e9, 2),
                   "gpu_event_basis": "HIP events recorded on the kernels' stream around the same K steps",
                   "fwd_us_avg": round(head["fwd_us_avg"], 3), "fwd_us_median": round(head["fwd_us_median"], 3),
                   "bwd_us_avg": round(head["bwd_us_avg"], 3), "bwd_us_median": round(head["bwd_us_median"], 3),
                   "event_launches_each": head["event_launches_each"],
                   "graph_replay_matches_eager": head["graph_replay_matches_eager"]},
        "copy_reference_GBs": round(copy_gbs, 1),
        "pct_of_copy_reference": round(100 * head["value_GBs"] / copy_gbs, 2),
        "warm": {"ms_per_step": round(head["warm_ms_per_step"], 6), "GBs": round(head["warm_GBs"], 1),
                 "cache_resident": head["warm_cache_resident"],
                 "note": "one buffer set repeated; not an HBM figure when cache_resident"},
        "roofline": {
            "kernel": fwd_k["kernel"],
            "bound": "hbm",
            "achieved": fwd_k["achieved"],
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": fwd_k["frac"],
            "traffic": fwd_k["traffic"],
            "kernels": kernels,
        },
        "cpu_baseline": None,
        "workloads": {},
    }
    if traffic is not None:
        line["roofline"]["traffic_detail"] = traffic
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(sp, w, j, src, sets[0].shards[0], args.cpu_seconds)
    del src, sets
    torch.cuda.empty_cache()
    if not args.no_secondary:
        for name, flags in SECONDARY:
            ws = W.WORKLOADS[name]
            shards = tuple(ws.shards)  # every shard the workload lists, one after another
            K2 = 40 if len(shards) > 2 else 400
            r, s2, st2 = measure(sp, ws, tuple(shards), K2, max(10, K2 // 10), stream, flags)
            label = name + ("+recompute_mask" if flags & sp.SP_FLAG_RECOMPUTE_MASK else "")
            line["workloads"][label] = {
                "shards_per_step": len(shards), "steps": K2,
                "GBs": round(r["value_GBs"], 1), "pct_of_peak": round(100 * r["value_GBs"] / PEAK_HBM_GBS, 2),
                "ms_per_step": round(r["ms_per_step"], 5), "tokens_per_s": round(r["tokens_per_s"], 1),
                "fwd_us": round(r["fwd_us_avg"], 2), "bwd_us": round(r["bwd_us_avg"], 2),
                "fwd_kernel_GBs": round(r["fwd_bytes"] / (r["fwd_us_avg"] * 1e-6) / 1e9, 1),
                "graph_replay_matches_eager": r["graph_replay_matches_eager"],
                "graph_replay_mismatch": r["graph_replay_mismatch"],
                "warm_GBs": round(r["warm_GBs"], 1), "warm_cache_resident": r["warm_cache_resident"],
            }
            del s2, st2
            torch.cuda.empty_cache()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
