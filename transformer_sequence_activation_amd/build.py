"""Build the HIP library libsp_region.so for gfx950 (MI355X), in-tree.

    python -m transformer_sequence_activation_amd.build [--resource-usage] [-D NAME=VALUE ...]
    python -m transformer_sequence_activation_amd.build --resource-table 'sp_fwd_kernel<1, 8, 512, 1, 512>;...'

The device code is compiled in a pass of its own, with packed fp32 instructions
(v_pk_add/mul/fma_f32) switched off; the host pass then embeds that code
object.  The feature exists only for the GPU target, so giving it to the host
pass as well would make the host compiler warn about an unknown feature.
"""
import argparse
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "sp_region.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsp_region.so")
ARCH = "gfx950"

COMMON = [f"--offload-arch={ARCH}", "-O3", "-std=c++17"]
# no packed fp32 instructions anywhere in the device code
DEVICE_ONLY = ["--cuda-device-only", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc():
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def _run(cmd, verbose, capture=False):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.run(cmd, check=True, capture_output=capture, text=capture)


def build(out=LIB, defines=(), resource_usage=False, verbose=False):
    """Compile csrc/sp_region.hip into `out`; always recompiles.  Returns the path.

    With resource_usage=True the compiler's kernel-resource remarks of the
    device pass are returned instead (the library is still built)."""
    defs = [f"-D{d}" for d in defines]
    fatbin = out + ".hipfb.tmp"
    tmp = out + ".tmp"
    dev = [_hipcc(), *COMMON, *DEVICE_ONLY, "-I", INCLUDE, *defs]
    if resource_usage:
        dev += ["-Rpass-analysis=kernel-resource-usage"]
    try:
        r = _run(dev + [SRC, "-o", fatbin], verbose, capture=resource_usage)
        host = [_hipcc(), *COMMON, "--cuda-host-only", "-fPIC", "-shared", "-I", INCLUDE, *defs,
                "-Xclang", "-fcuda-include-gpubinary", "-Xclang", fatbin, SRC, "-o", tmp]
        _run(host, verbose)
        os.replace(tmp, out)
    finally:
        for f in (fatbin, tmp):
            if os.path.exists(f):
                os.remove(f)
    return r.stderr if resource_usage else out


def resource_table(out, kernels=None):
    """Build `out` with the compiler's kernel-resource remarks and return a text
    table (kernel, VGPRs, AGPRs, SGPRs, spills, scratch, LDS, waves per SIMD),
    keeping kernels whose demangled name contains one of `kernels`."""
    stderr = build(out, resource_usage=True)
    rows, cur = [], None
    keys = {"VGPRs": "vgpr", "AGPRs": "agpr", "TotalSGPRs": "sgpr", "VGPRs Spill": "vspill",
            "ScratchSize [bytes/lane]": "scratch", "LDS Size [bytes/block]": "lds",
            "Occupancy [waves/SIMD]": "occ"}
    for line in stderr.splitlines():
        if "remark:" not in line:
            continue
        body = line.split("remark:", 1)[1].split("[-Rpass", 1)[0].strip()
        if body.startswith("Function Name:"):
            cur = {"name": body.split(":", 1)[1].strip()}
            rows.append(cur)
        elif cur is not None and ":" in body:
            k, v = body.split(":", 1)
            if k.strip() in keys:
                cur[keys[k.strip()]] = v.strip()
    names = subprocess.run(["c++filt"], input="\n".join(x["name"] for x in rows), capture_output=True,
                           text=True).stdout.splitlines()
    out_lines = [f"{'kernel':<92} {'VGPR':>5} {'AGPR':>5} {'SGPR':>5} {'spill':>5} {'scratch':>7} "
                 f"{'LDS':>6} {'waves/SIMD':>10}"]
    for x, n in zip(rows, names):
        n = n.replace("(anonymous namespace)::", "").replace("void ", "").split("(", 1)[0]
        if kernels and not any(k in n for k in kernels):
            continue
        out_lines.append(f"{n:<92} {x.get('vgpr', '?'):>5} {x.get('agpr', '?'):>5} {x.get('sgpr', '?'):>5} "
                         f"{x.get('vspill', '?'):>5} {x.get('scratch', '?'):>7} {x.get('lds', '?'):>6} "
                         f"{x.get('occ', '?'):>10}")
    return "\n".join(out_lines)


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=LIB)
    ap.add_argument("-D", dest="defines", action="append", default=[])
    ap.add_argument("--resource-table", metavar="KERNELS", default=None,
                    help="build and print the resource table of the kernels whose names contain one "
                         "of these ';'-separated substrings ('' = all)")
    args = ap.parse_args()
    if args.resource_table is not None:
        print(resource_table(args.out, [k for k in args.resource_table.split(";") if k]))
        raise SystemExit(0)
    print(build(args.out, args.defines, verbose=True))
