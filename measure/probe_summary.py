"""Markdown summaries of the measurement probes' JSON lines.

    ./measure/stream_probe > stream_probe.jsonl
    python -m measure.probe_summary stream stream_probe.jsonl > profiles/stream_probe_mi355x.md
    ./measure/sync_probe > sync_probe.jsonl
    python -m measure.probe_summary sync sync_probe.jsonl > profiles/sync_probe_mi355x.md
"""
import argparse
import json

MIB = 1 << 20


def _rows(path):
    with open(path) as f:
        return [json.loads(line) for line in f if line.startswith("{")]


def _stream_size(r):
    if r["probe"] == "copy":
        return f"{r['bytes_each_way'] // MIB} MiB each way"
    return f"{r['stream_bytes'] // MIB} MiB per stream"


def _stream_name(r):
    return r["probe"] + (f" T={r['T']}" if "T" in r else "")


def _policy(nt):
    return "nt" if nt else "cached"


def stream(path):
    rows = _rows(path)
    best = {}
    for r in rows:
        if r["probe"] == "copy":
            continue
        key = (_stream_name(r), _stream_size(r))
        if key not in best or r["us"] < best[key]["us"]:
            best[key] = r
    out = [
        "# Streaming-bandwidth ceilings on MI355X (gfx950) -- measure/stream_probe",
        "",
        "Kernels that only move bytes, timed with hipEvents over 60 back-to-back launches, each on a buffer set of its",
        "own where the 1 GiB buffers allow (0.8 to 1.3 GB cycled, more than the 256 MB Infinity Cache, so every launch",
        "reads HBM).  `copy` is a grid-stride 16-byte nontemporal copy.  `fwd_pattern` / `bwd_pattern`",
        "have exactly the SP forward's / backward's memory pattern (T partial streams + residual read, h / y / mask",
        "written; dY / h / mask read, d_residual / dP written) with no arithmetic, at the stream sizes of the",
        "LayerNorm T=8 H=4096 shard (4 MiB per stream), the MiniMind T=2 shard (3 MiB) and the large-hidden T=8",
        "H=8192 B=2 shard (32 MiB), swept over chunks per lane, workgroup size and the cache policy of loads and",
        "stores (nt = nontemporal).  A workgroup of BLOCK lanes takes BLOCK x chunks consecutive 16-byte chunks.",
        "",
        "## Command",
        "",
        "```",
        "python -m measure.build",
        "./measure/stream_probe > stream_probe.jsonl",
        "python -m measure.probe_summary stream stream_probe.jsonl > profiles/stream_probe_mi355x.md",
        "```",
        "",
        "## Best pattern per case (the ceilings the SP kernels are compared with)",
        "",
        "| pattern | size | us | GB/s (read+write) | launch shape |",
        "|---|---|---|---|---|",
    ]
    for key in sorted(best):
        r = best[key]
        out.append(f"| {key[0]} | {key[1]} | {r['us']:.2f} | {r['GBs']:.0f} | {r['chunks_per_lane']} chunk(s) per lane, "
                   f"{r['block']}-lane workgroups, {_policy(r['nt_loads'])} loads, {_policy(r['nt_stores'])} stores |")
    out += ["", "## Every measurement", "",
            "| probe | size | launch shape | loads / stores | us | GB/s |", "|---|---|---|---|---|---|"]
    for r in rows:
        if r["probe"] == "copy":
            shape, pol = f"grid {r['grid']}", ""
        else:
            shape = f"{r['chunks_per_lane']} chunk(s) x {r['block']} lanes, grid {r['grid']}"
            pol = f"{_policy(r['nt_loads'])} / {_policy(r['nt_stores'])}"
        out.append(f"| {_stream_name(r)} | {_stream_size(r)} | {shape} | {pol} | {r['us']:.2f} | {r['GBs']:.0f} |")
    return "\n".join(out) + "\n"


def sync(path):
    rows = _rows(path)
    out = [
        "# Cost of workgroups of one launch waiting for each other on MI355X (gfx950) -- measure/sync_probe",
        "",
        "What a kernel pays when a token row is split over several workgroups (they must exchange partial row sums",
        "before finishing the row) or when a reduction over workgroups is finished inside the launch (the last",
        "workgroup to arrive reads everyone's partials) instead of by a second launch.  Every wait in the probe is",
        "bounded and every grid fits the device at once.",
        "",
        "## Command",
        "",
        "```",
        "python -m measure.build",
        "./measure/sync_probe > sync_probe.jsonl",
        "python -m measure.probe_summary sync sync_probe.jsonl > profiles/sync_probe_mi355x.md",
        "```",
        "",
        "## Results",
        "",
        "| measurement | time |",
        "|---|---|",
    ]
    for r in rows:
        p = r["probe"]
        if p == "empty_kernel":
            out.append(f"| empty kernel, {r['grid']} workgroup(s), back to back | {r['us']:.2f} us per launch |")
        elif p == "atomic_roundtrip":
            out.append(f"| one device-scope atomic add waiting for the previous one | {r['ns']:.0f} ns |")
        elif p == "group_barrier":
            out.append(f"| {r['workgroups']} workgroups, groups of {r['group']}, {r['steps']} exchange step(s) "
                       f"(waits given up: {r['waits_given_up']}) | {r['us']:.2f} us per launch |")
        elif p == "last_arriver":
            out.append(f"| {r['workgroups']} workgroups store {r['floats_each']} floats each; the last to arrive "
                       f"reads them all | {r['store_only_us']:.2f} us without the read, "
                       f"{r['with_last_arriver_read_us']:.2f} us with it |")
    return "\n".join(out) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("probe", choices=("stream", "sync"))
    ap.add_argument("jsonl")
    a = ap.parse_args()
    print(stream(a.jsonl) if a.probe == "stream" else sync(a.jsonl), end="")


if __name__ == "__main__":
    main()
