"""Build the measurement probes (measure/stream_probe.hip, measure/sync_probe.hip) for gfx950.

    python -m measure.build        # writes measure/stream_probe and measure/sync_probe

A measurement tool beside bench.py and profiles/, not part of the library.
Like the library, the device code is compiled in a pass of its own with packed
fp32 instructions switched off, and the host pass embeds it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
PROBES = ("stream_probe", "sync_probe")


def build(name, verbose=True):
    src = os.path.join(HERE, name + ".hip")
    out = os.path.join(HERE, name)
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    common = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17"]
    fatbin, tmp = out + ".hipfb.tmp", out + ".tmp"
    cmds = [common + ["--cuda-device-only", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                      src, "-o", fatbin],
            common + ["--cuda-host-only", "-Xclang", "-fcuda-include-gpubinary", "-Xclang", fatbin, src,
                      "-o", tmp]]
    try:
        for cmd in cmds:
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    finally:
        for f in (fatbin, tmp):
            if os.path.exists(f):
                os.remove(f)
    return out


if __name__ == "__main__":
    for name in PROBES:
        print(build(name))
