"""Markdown summaries of rocprofv3 runs of the SP-region kernels (the files in profiles/).

Input: the text that measure.rocprof_summary prints for each results database,
and the traffic JSON it writes.  The commands that produce them are repeated in
each summary.

    python -m measure.profile_report kernels WORKLOAD KT.txt PMC.txt TRAFFIC.json DIGEST
    python -m measure.profile_report bench KT_BENCH.txt DIGEST
    python -m measure.profile_report sq WORKLOAD PASS1.txt PASS2.txt DIGEST
"""
import argparse
import json
import re
import sys

PMC1 = ("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU",
        "SQ_ACTIVE_INST_VMEM", "SQ_INSTS_VALU", "SQ_INSTS_VMEM_RD")
PMC2 = ("SQ_INSTS_VMEM_WR", "SQ_ACTIVE_INST_LDS", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_INST_LEVEL_VMEM",
        "SQ_INST_CYCLES_VMEM_RD", "SQ_WAVES", "SQ_INSTS_SALU")


def _read(path):
    with open(path) as f:
        return f.read().strip()


def describe(name):
    """One line on the workload's shard and the backward's dgamma schedule (host-side planner)."""
    import transformer_sequence_activation_amd as sp
    from transformer_sequence_activation_amd import workloads as W
    w = W.WORKLOADS[name]
    j = w.shards[-1] if len(w.shards) == 1 else w.shards[0]
    sp.load()
    d = sp.make_desc(w.S, w.B, w.H, w.T, j, w.dtype, w.norm, w.eps, w.p, w.seed)
    k = sp.sp_region_bwd_schedule(d)
    norm = "LayerNorm" if w.norm == "ln" else "RMSNorm"
    rows = (w.S // w.T) * w.B
    if k == 0:
        sched = "the partial-row schedule (main kernel + dgamma finish kernel)"
    elif k == 1:
        sched = f"the column schedule for dgamma/dbeta (one segment of all {rows} rows)"
    else:
        sched = f"the column schedule with {k} row segments per strip"
    return (f"{norm}, T={w.T}, [S,B,H] = [{w.S},{w.B},{w.H}], shard {j} ({rows} rows); "
            f"the backward takes {sched}.")


def kernels(name, kt, pmc, traffic, digest):
    tr = json.load(open(traffic))
    mb = lambda x: f"{x / 1e6:.2f} MB"
    pmc_text = "\n".join(line for line in _read(pmc).splitlines() if not line.startswith("wrote "))
    return f"""# SP-region kernels on the {name} shard -- rocprofv3 summary

{describe(name)}
Kernel source digest (sha256 of transformer_sequence_activation_amd/csrc/sp_region.hip, first 16 hex): `{digest}`.
Hardware: MI355X (gfx950, 256 CUs), ROCm 7.2, one GPU.

## Commands (REPO = the repository root, on the MI355X machine)

```
cd /tmp && export TMPDIR=/tmp
rocprofv3 --kernel-trace --stats -d /tmp/kt_{name} -o kt -- python3 $REPO/bench.py --profile-pass --workload {name}
timeout -s KILL 180 rocprofv3 --pmc FETCH_SIZE -d /tmp/pmc_FETCH_SIZE_{name} -o pmc -- python3 $REPO/bench.py --profile-pass --workload {name}
timeout -s KILL 180 rocprofv3 --pmc WRITE_SIZE -d /tmp/pmc_WRITE_SIZE_{name} -o pmc -- python3 $REPO/bench.py --profile-pass --workload {name}
cd $REPO
python3 -m measure.rocprof_summary /tmp/kt_{name}/kt_results.db --filter sp_ > kt.txt
python3 -m measure.rocprof_summary /tmp/pmc_FETCH_SIZE_{name}/pmc_results.db /tmp/pmc_WRITE_SIZE_{name}/pmc_results.db --copy-bytes 268435456 --filter sp_ --traffic-json profiles/traffic_{name}.json --source-digest {digest} > pmc.txt
python3 -m measure.profile_report kernels {name} kt.txt pmc.txt profiles/traffic_{name}.json {digest} > profiles/sp_region_kernels_{name}.md
```

`bench.py --profile-pass` launches a 256 MiB device copy three times, then forward + backward once on each
rotating buffer set (more than 1.5 GB of sets, so every launch reads HBM), three times over.

## Kernel durations (kernel trace)

```
{_read(kt)}
```

## HBM bytes per dispatch (FETCH_SIZE, WRITE_SIZE)

FETCH_SIZE and WRITE_SIZE count L2-to-fabric traffic (Infinity Cache hits included).  On gfx950 FETCH_SIZE
of a copy reads half of the bytes copied, so both counters are scaled by what they read for the 256 MiB copy
in the same run (the calibration line).

```
{pmc_text}
```

Per launch: forward fetch {mb(tr['fwd_fetch_bytes'])}, write {mb(tr['fwd_write_bytes'])};
backward main kernel fetch {mb(tr['bwd_main_fetch_bytes'])}, write {mb(tr['bwd_main_write_bytes'])};
finish kernel fetch {mb(tr['bwd_finish_fetch_bytes'])}, write {mb(tr['bwd_finish_write_bytes'])}.
"""


def bench(kt, digest):
    return f"""# bench.py under a kernel trace -- LayerNorm T=8 H=4096 shard 3 (the headline workload)

Kernel source digest: `{digest}`.  MI355X (gfx950), one GPU.

## Commands

```
cd /tmp && export TMPDIR=/tmp
rocprofv3 --kernel-trace --stats -d /tmp/kt_bench -o kt -- python3 $REPO/bench.py --no-cpu-baseline --no-secondary --steps 400 --warmup 40
cd $REPO && python3 -m measure.rocprof_summary /tmp/kt_bench/kt_results.db --filter sp_ > kt_bench.txt
python3 -m measure.profile_report bench kt_bench.txt {digest} > profiles/bench_kernel_trace_layernorm_T8_S4096_B1_H4096.md
```

## Kernel durations over the whole bench run (warm-up, graph check, timed steps, event pass)

Every launch of the run is counted: eager launches on 20 rotating buffer sets, the graph replays of the
replay check, the timed steps and the event-timed launch pass.

```
{_read(kt)}
```
"""


def _counters(path):
    """{kernel: {counter: median per dispatch}} from a rocprof_summary counter table."""
    out = {}
    for line in _read(path).splitlines():
        m = re.match(r"(sp_\S+.*?>)\s+(SQ_\w+)\s+(\d+)\s+([\d.]+)", line)
        if m:
            out.setdefault(m.group(1), {})[m.group(2)] = float(m.group(4))
    return out


def sq(name, pass1, pass2, digest):
    c = _counters(pass1)
    for k, v in _counters(pass2).items():
        c.setdefault(k, {}).update(v)
    cmd = "\n".join([
        "cd /tmp && export TMPDIR=/tmp",
        f"timeout -s KILL 120 rocprofv3 --pmc {' '.join(PMC1)} -d /tmp/sq1 -o pmc -- python3 $REPO/bench.py "
        f"--profile-pass --workload {name}",
        f"timeout -s KILL 120 rocprofv3 --pmc {' '.join(PMC2)} -d /tmp/sq2 -o pmc -- python3 $REPO/bench.py "
        f"--profile-pass --workload {name}",
        "cd $REPO",
        "python3 -m measure.rocprof_summary /tmp/sq1/pmc_results.db --filter sp_ > sq1.txt",
        "python3 -m measure.rocprof_summary /tmp/sq2/pmc_results.db --filter sp_ > sq2.txt",
        f"python3 -m measure.profile_report sq {name} sq1.txt sq2.txt {digest} > profiles/sq_counters_{name}.md",
    ])
    out = [f"# Instruction and wait counters of the {name} shard kernels (SQ, gfx950)", "",
           f"Kernel source digest: `{digest}`.  Two `rocprofv3 --pmc` passes of eight SQ counters each over",
           "`bench.py --profile-pass` (forward + backward once on each of the rotating buffer sets, three times over;",
           "medians per dispatch).  The SQ wave counters count in units of 4 cycles, the time one wave64 VALU",
           "instruction occupies a 16-lane SIMD: SQ_ACTIVE_INST_VALU equals SQ_INSTS_VALU.",
           "", "## Commands (REPO = the repository root, on the MI355X machine)", "", "```", cmd, "```", "",
           "## Per wave (medians per dispatch divided by SQ_WAVES)", "",
           "| kernel | waves | resident (4-cycle units) | VALU instructions | VALU share of residency | "
           "waiting on a dependency (SQ_WAIT_INST_ANY) | waiting, any cause (SQ_WAIT_ANY) | vector loads | "
           "vector stores | LDS instructions | scalar instructions |",
           "|---|---|---|---|---|---|---|---|---|---|---|"]
    conflicts = []
    for k, v in c.items():
        w, wc = v["SQ_WAVES"], v["SQ_WAVE_CYCLES"]
        out.append(f"| `{k}` | {int(w)} | {wc / w:.0f} | {v['SQ_INSTS_VALU'] / w:.0f} | "
                   f"{100 * v['SQ_INSTS_VALU'] / wc:.1f}% | {100 * v['SQ_WAIT_INST_ANY'] / wc:.1f}% | "
                   f"{100 * v['SQ_WAIT_ANY'] / wc:.1f}% | {v['SQ_INSTS_VMEM_RD'] / w:.1f} | "
                   f"{v['SQ_INSTS_VMEM_WR'] / w:.1f} | {v['SQ_INSTS_LDS'] / w:.1f} | {v['SQ_INSTS_SALU'] / w:.0f} |")
        conflicts.append(f"`{k.split('<')[0]}` {v['SQ_LDS_BANK_CONFLICT']:.0f}")
    out += ["", "LDS bank conflicts per dispatch: " + ", ".join(conflicts) + ".", "", "## Raw summaries", "", "```"]
    out += [line.rstrip() for line in _read(pass1).splitlines()
            if "sp_" in line or line.startswith("kernel") or line.startswith("#")]
    out += [line.rstrip() for line in _read(pass2).splitlines() if "sp_" in line]
    out += ["```"]
    return "\n".join(out) + "\n"


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    k = sub.add_parser("kernels")
    for arg in ("workload", "kernel_trace", "counters", "traffic", "digest"):
        k.add_argument(arg)
    b = sub.add_parser("bench")
    b.add_argument("kernel_trace")
    b.add_argument("digest")
    q = sub.add_parser("sq")
    for arg in ("workload", "pass1", "pass2", "digest"):
        q.add_argument(arg)
    a = ap.parse_args()
    if a.what == "kernels":
        text = kernels(a.workload, a.kernel_trace, a.counters, a.traffic, a.digest)
    elif a.what == "bench":
        text = bench(a.kernel_trace, a.digest)
    else:
        text = sq(a.workload, a.pass1, a.pass2, a.digest)
    sys.stdout.write(text)


if __name__ == "__main__":
    main()
