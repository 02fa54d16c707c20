"""Build the streaming-bandwidth probe (measure/stream_probe.hip) for gfx950.

    python -m measure.build        # writes measure/stream_probe

A measurement tool beside bench.py and profiles/, not part of the library.
Like the library, the device code is compiled in a pass of its own with packed
fp32 instructions switched off, and the host pass embeds it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "stream_probe.hip")
PROBE = os.path.join(HERE, "stream_probe")


def build(out=PROBE, verbose=True):
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    common = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17"]
    fatbin, tmp = out + ".hipfb.tmp", out + ".tmp"
    cmds = [common + ["--cuda-device-only", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                      SRC, "-o", fatbin],
            common + ["--cuda-host-only", "-Xclang", "-fcuda-include-gpubinary", "-Xclang", fatbin, SRC,
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
    print(build())
