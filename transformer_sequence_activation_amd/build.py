"""Build the HIP library libsp_region.so for gfx950 (MI355X), in-tree.

    python -m transformer_sequence_activation_amd.build [--resource-usage] [-D NAME=VALUE ...]
"""
import argparse
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "sp_region.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsp_region.so")
PROBE_SRC = os.path.join(PKG, "csrc", "stream_probe.hip")
PROBE = os.path.join(PKG, "stream_probe")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed fp32 instructions (v_pk_add/mul/fma_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(out=LIB, defines=(), resource_usage=False, verbose=False):
    """Compile csrc/sp_region.hip into `out`; always recompiles.  Returns the path."""
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    cmd = [hipcc, *HIPCC_FLAGS, "-I", INCLUDE]
    cmd += [f"-D{d}" for d in defines]
    if resource_usage:
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    tmp = out + ".tmp"
    cmd += [SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_probe(out=PROBE, verbose=False):
    """Compile the streaming-bandwidth probe executable; always recompiles."""
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    flags = [f for f in HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    tmp = out + ".tmp"
    cmd = [hipcc, *flags, PROBE_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=LIB)
    ap.add_argument("-D", dest="defines", action="append", default=[])
    ap.add_argument("--resource-usage", action="store_true")
    ap.add_argument("--probe", action="store_true", help="also build the stream_probe executable")
    args = ap.parse_args()
    print(build(args.out, args.defines, args.resource_usage, verbose=True))
    if args.probe:
        print(build_probe(verbose=True))
