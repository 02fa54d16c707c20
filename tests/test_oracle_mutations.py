"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of oracle/sp_oracle.c -- a dropped term,
a wrong sign, constant, index or operand -- builds the copy in a temporary
directory and runs tests/test_oracle_pins.py against it.  The pins must fail.
The repository's own oracle is not touched.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = [
    ("dropped LayerNorm mean term in the backward",
     "dh = rs * (g[k] - c1 - xhat[k] * c2);", "dh = rs * (g[k] - xhat[k] * c2);"),
    ("wrong Philox key increment",
     "PHILOX_WEYL0 = 0x9E3779B9u;", "PHILOX_WEYL0 = 0x9E3779B7u;"),
    ("wrong output word of the generator",
     "return out[gi & 3u];", "return out[(gi + 1) & 3u];"),
    ("mask keyed on the shard-local index",
     "uint64_t gi = (uint64_t)((d->j * R + row0 + r) * H + k);",
     "uint64_t gi = (uint64_t)((row0 + r) * H + k);"),
    ("dgamma from dY * gamma instead of dY",
     "dgamma[k] += dy * xhat[k];", "dgamma[k] += g[k] * xhat[k];"),
    ("unbiased LayerNorm variance",
     "var = sumsq / (double)H;", "var = sumsq / (double)(H - 1);"),
    ("dP without the 1/(1-p) scale",
     "mask[i] ? dh * scale : 0.0", "mask[i] ? dh : 0.0"),
    ("last partial skipped in the sum",
     "for (t = 1; t < d->T; ++t) acc = acc + (float)load_elem(P[t], i, d->dtype);",
     "for (t = 1; t < d->T - 1; ++t) acc = acc + (float)load_elem(P[t], i, d->dtype);"),
    ("bf16 by truncation instead of round-to-nearest-even",
     "u += 0x7FFFu + ((u >> 16) & 1u);", "u += 0u;"),
    ("fp32-mode partials summed in double",
     "float acc = (float)load_elem(P[0], i, d->dtype);", "double acc = (double)load_elem(P[0], i, d->dtype);"),
    ("fp32-mode backward scaled by the double 1/(1-p)",
     "if (d->dtype != SPO_F64) scale = (double)(float)scale;",
     "if (d->dtype == SPO_BF16) scale = (double)(float)scale;"),
    ("LayerNorm bias added with the wrong sign",
     "gamma[k] * ((hrow[k] - mu) * rs) + beta[k]", "gamma[k] * ((hrow[k] - mu) * rs) - beta[k]"),
]


def run_pins_on_copy(tmp_path, old=None, new=None):
    """Copy the oracle and its pins, optionally replace `old` by `new` in the
    C source, build, run the pins; returns the pytest run."""
    src = open(os.path.join(ROOT, "oracle", "sp_oracle.c")).read()
    if old is not None:
        assert src.count(old) == 1, f"the text to mutate is not unique in the oracle: {old}"
        src = src.replace(old, new)
    work = tmp_path / "copy"
    shutil.copytree(os.path.join(ROOT, "oracle"), work / "oracle",
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    (work / "tests").mkdir()
    for f in ("conftest.py", "test_oracle_pins.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), work / "tests" / f)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), work / "tests" / "golden")
    (work / "oracle" / "sp_oracle.c").write_text(src)
    subprocess.run([sys.executable, os.path.join("oracle", "build.py")], cwd=work, check=True,
                   capture_output=True)
    return subprocess.run([sys.executable, "-m", "pytest", os.path.join("tests", "test_oracle_pins.py"),
                           "-x", "-q", "-p", "no:cacheprovider"], cwd=work, capture_output=True, text=True,
                          timeout=600)


def test_unchanged_copy_passes(tmp_path):
    r = run_pins_on_copy(tmp_path)
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(tmp_path, name, old, new):
    r = run_pins_on_copy(tmp_path, old, new)
    # 1 = some test failed; 0 would mean the mistake went unnoticed, >1 a broken run
    assert r.returncode == 1, f"{name}: pins returned {r.returncode}\n{r.stdout[-2000:]}"
