"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test ties one part of oracle/sp_oracle.c to something the oracle does not
compute itself: the pages' worked example and printed numbers, an independent
library implementation (PyTorch's header Philox engine, torch's bf16 cast,
torch's rms_norm / layer_norm / dropout / autograd), closed-form invariants,
binomial bounds, or central finite differences.
"""
import math
import os
import subprocess
import tempfile

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import ring_rs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def desc(S, B, H, T, j, dtype, norm, eps, p, seed=1234):
    return oracle.make_desc(S, B, H, T, j, dtype, norm, eps, p, seed)


def shard_rows(full, S, B, H, T, j):
    N = (S // T) * B * H
    return np.ascontiguousarray(full.reshape(-1)[j * N:(j + 1) * N]).reshape(-1, H)


# ---------------------------------------------------------------------------
# Philox4x32-10 against PyTorch's header-only engine (an independent
# implementation of the SC'11 generator).  The engine started at
# (seed, subsequence 0, offset o) emits, call by call, the four words of
# counter (o, 0) then (o+1, 0), ... -- exactly the per-element words the
# oracle assigns to global indices 4*o, 4*o+1, ...

_PHILOX_PROBE = r"""
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
#include <cstdlib>
#include <cstdint>
int main(int argc, char** argv) {
  uint64_t seed = strtoull(argv[1], nullptr, 10);
  uint64_t offset = strtoull(argv[2], nullptr, 10);
  long n = atol(argv[3]);
  at::philox_engine eng(seed, 0, offset);
  for (long i = 0; i < n; ++i) { uint32_t u = eng(); fwrite(&u, 4, 1, stdout); }
  return 0;
}
"""


@pytest.fixture(scope="module")
def philox_probe():
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    if not os.path.exists(os.path.join(inc, "ATen", "core", "PhiloxRNGEngine.h")):
        pytest.skip("PyTorch's PhiloxRNGEngine.h header is not installed")
    d = tempfile.mkdtemp()
    src = os.path.join(d, "probe.cpp")
    exe = os.path.join(d, "probe")
    with open(src, "w") as f:
        f.write(_PHILOX_PROBE)
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", inc, src, "-o", exe], check=True)
    return exe


def _engine_words(exe, seed, offset, n):
    out = subprocess.run([exe, str(seed), str(offset), str(n)], check=True, capture_output=True)
    return np.frombuffer(out.stdout, dtype=np.uint32)


@pytest.mark.parametrize("seed,offset,n", [
    (1234, 0, 1 << 20),                     # the masks' seed, first 2^20 words
    (0, 0, 4096),
    (0xFFFFFFFFFFFFFFFF, 0, 4096),          # both key words all ones
    (0x0123456789ABCDEF, (1 << 32) - 3, 64),  # counter crosses into its high word
    (42, 123456789012, 256),
])
def test_philox_matches_torch_header_engine(philox_probe, seed, offset, n):
    ref = _engine_words(philox_probe, seed, offset, n)
    got = oracle.uniform_words(seed, 4 * offset, n)
    assert np.array_equal(got, ref)


def test_keep_mask_p0_keeps_everything():
    assert oracle.keep_mask(1234, 0.0, 0, 100000).all()


# Keep count within N(1-p) +- 5 sqrt(N p (1-p)) for the shards the workloads use
# (the fifth workload: its first and last shard).
@pytest.mark.parametrize("S,B,H,T,j", [
    (256, 1, 64, 2, 0),
    (2048, 2, 768, 2, 0), (2048, 2, 768, 2, 1),
    (4096, 1, 4096, 8, 3),
    (8192, 2, 8192, 8, 5),
    (32768, 1, 8192, 8, 0), (32768, 1, 8192, 8, 7),
])
def test_keep_fraction_within_binomial_bounds(S, B, H, T, j):
    p = np.float32(0.1)
    N = (S // T) * B * H
    m = oracle.keep_mask(1234, float(p), j * N, N)
    k = int(m.sum())
    mean = N * (1 - float(p))
    sd = math.sqrt(N * float(p) * (1 - float(p)))
    assert abs(k - mean) <= 5 * sd, (k, mean, sd)


# ---------------------------------------------------------------------------
# bf16 rounding against torch's cast.

def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    ties = (rng.integers(0, 2**16, size=4096, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    special = np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 3.3895314e38, 1e-40, -1e-45,
                        1.00390625, 1.01171875, 65504.0], np.float32)
    x = np.concatenate([vals, ties, special])
    got = oracle.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all(np.isnan(oracle.bf16_to_f32(got[nan])))


# ---------------------------------------------------------------------------
# The reduce-scatter: the pages' worked example and all-reduce = RS + AG.

def _golden_ring_tables():
    tables, cur = [], None
    with open(os.path.join(GOLDEN, "ring_reduce_scatter_T4.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("step"):
                cur = []
                tables.append(cur)
            else:
                cur.append(line.split())
    return tables


def test_ring_reduce_scatter_reproduces_worked_example():
    assert ring_rs.symbolic_tables(4) == _golden_ring_tables()
    _, sent = ring_rs.simulate([[np.zeros(1)] * 4 for _ in range(4)])
    assert sent == [3, 3, 3, 3]  # (T-1) blocks of N/T each per rank


@pytest.mark.parametrize("T", [2, 3, 4, 8])
def test_allreduce_equals_reduce_scatter_plus_all_gather(T):
    """concat_j sum_t P_t^(j) == sum_t P_t, on integer values the fp32 sums carry exactly."""
    S, B, H = 8 * T, 2, 32
    rng = np.random.default_rng(T)
    P_int = rng.integers(-31, 32, size=(T, S, B, H))
    P = [oracle.f32_to_bf16(P_int[t].astype(np.float32)) for t in range(T)]
    exact = P_int.sum(axis=0).reshape(-1)
    zeros = np.zeros((S // T * B, H), np.uint16)
    gam = np.ones(H)
    hs = []
    for j in range(T):
        d = desc(S, B, H, T, j, oracle.BF16, oracle.RMSNORM, 1e-6, 0.0)
        out = oracle.fwd(d, [shard_rows(P[t], S, B, H, T, j) for t in range(T)], zeros, gam)
        hs.append(oracle.bf16_to_f32(out["h"]).reshape(-1))
    got = np.concatenate(hs)
    # |sum| <= 31*T <= 248: every integer up to 256 is exact in bf16
    assert np.array_equal(got.astype(np.int64), exact)
    # the ring simulator gives the same blocks
    blocks = [[P_int[t].reshape(T, -1)[c] for c in range(T)] for t in range(T)]
    table, _ = ring_rs.simulate(blocks)
    ring = np.concatenate([table[j][j] for j in range(T)])
    assert np.array_equal(ring, exact)


@pytest.mark.parametrize("T,norm", [(2, oracle.RMSNORM), (4, oracle.LAYERNORM), (8, oracle.RMSNORM)])
def test_shards_concatenate_to_the_unsharded_run(T, norm):
    """Real-valued fp32 data with dropout: the T shards' h, y and mask,
    concatenated, are bit-identical to one unsharded run (T = 1) fed the fp32
    sum of the partials taken in the same order -- concat_j sum_t P_t^(j) equals
    sum_t P_t, and the rest of the region is per element and per token row."""
    S, B, H = 8 * T, 2, 24
    rng = np.random.default_rng(40 + T)
    P = [(rng.standard_normal((S, B, H)) / math.sqrt(T)).astype(np.float32) for _ in range(T)]
    res = rng.standard_normal((S, B, H)).astype(np.float32)
    gam = 1 + 0.02 * rng.standard_normal(H)
    bet = 0.02 * rng.standard_normal(H) if norm == oracle.LAYERNORM else None
    eps = 1e-5 if norm == oracle.LAYERNORM else 1e-6
    total = P[0].copy()
    for t in range(1, T):
        total = total + P[t]  # fp32 adds in t order
    one = oracle.fwd(desc(S, B, H, 1, 0, oracle.F32, norm, eps, 0.25), [total.reshape(-1, H)],
                     res.reshape(-1, H), gam, bet)
    parts = {k: [] for k in ("h", "y", "mask")}
    for j in range(T):
        d = desc(S, B, H, T, j, oracle.F32, norm, eps, 0.25)
        out = oracle.fwd(d, [shard_rows(P[t], S, B, H, T, j) for t in range(T)],
                         shard_rows(res, S, B, H, T, j), gam, bet)
        for k in parts:
            parts[k].append(out[k])
    for k in parts:
        assert np.array_equal(np.concatenate(parts[k]), one[k]), k


def test_mask_is_keyed_on_the_global_index():
    """Shard masks for any T tile the mask of the whole tensor (the mask must
    correspond along the sequence whatever the split)."""
    S, B, H = 64, 2, 48
    full = oracle.keep_mask(1234, 0.3, 0, S * B * H)
    rng = np.random.default_rng(3)
    for T in (1, 2, 4, 8):
        P = [oracle.f32_to_bf16(rng.standard_normal((S, B, H)).astype(np.float32)) for _ in range(T)]
        res = oracle.f32_to_bf16(rng.standard_normal((S, B, H)).astype(np.float32))
        parts = []
        for j in range(T):
            d = desc(S, B, H, T, j, oracle.BF16, oracle.RMSNORM, 1e-6, 0.3)
            out = oracle.fwd(d, [shard_rows(P[t], S, B, H, T, j) for t in range(T)],
                             shard_rows(res, S, B, H, T, j), np.ones(H))
            parts.append(out["mask"].reshape(-1))
        assert np.array_equal(np.concatenate(parts), full)


def test_row_blocks_tile_the_shard():
    """Running rows [a, b) alone gives the same rows as the whole shard."""
    S, B, H, T, j = 32, 3, 40, 4, 2
    rng = np.random.default_rng(11)
    P = [oracle.f32_to_bf16(rng.standard_normal((S, B, H)).astype(np.float32)) for _ in range(T)]
    res = oracle.f32_to_bf16(rng.standard_normal((S, B, H)).astype(np.float32))
    gam = 1 + 0.02 * rng.standard_normal(H)
    bet = 0.02 * rng.standard_normal(H)
    d = desc(S, B, H, T, j, oracle.BF16, oracle.LAYERNORM, 1e-5, 0.2)
    Ps = [shard_rows(P[t], S, B, H, T, j) for t in range(T)]
    rs = shard_rows(res, S, B, H, T, j)
    whole = oracle.fwd(d, Ps, rs, gam, bet)
    a, b = 5, 17
    part = oracle.fwd(d, [x[a:b] for x in Ps], rs[a:b], gam, bet, row0=a, nrows=b - a)
    for k in ("h", "y", "mask", "mean", "rstd"):
        assert np.array_equal(part[k], whole[k][a:b]), k


# ---------------------------------------------------------------------------
# Norm forward: invariants and the library routines.

def _f64_case(S, B, H, T, j, seed, outlier=False):
    rng = np.random.default_rng(seed)
    P = [rng.standard_normal((S, B, H)) / math.sqrt(T) for _ in range(T)]
    if outlier:
        P[0][0, 0, :] *= 100.0
    res = rng.standard_normal((S, B, H))
    gam = 1 + 0.02 * rng.standard_normal(H)
    bet = 0.02 * rng.standard_normal(H)
    return P, res, gam, bet


@pytest.mark.parametrize("eps", [0.0, 1e-6, 1e-2])
def test_rmsnorm_output_has_unit_rms(eps):
    S, B, H, T, j = 16, 2, 96, 2, 1
    P, res, _, _ = _f64_case(S, B, H, T, j, 5)
    d = desc(S, B, H, T, j, oracle.F64, oracle.RMSNORM, eps, 0.1)
    out = oracle.fwd(d, [shard_rows(x, S, B, H, T, j) for x in P], shard_rows(res, S, B, H, T, j),
                     np.ones(H))
    eps = float(np.float32(eps))  # the descriptor carries eps as fp32
    ms = np.mean(out["h"] ** 2, axis=1)
    rms_y = np.sqrt(np.mean(out["y"] ** 2, axis=1))
    # exactly sqrt(ms/(ms+eps)): 1 at eps = 0, within eps/(2 ms) of 1 otherwise
    assert np.allclose(rms_y, np.sqrt(ms / (ms + eps)), rtol=1e-13, atol=0)
    assert np.all(np.abs(rms_y - 1) <= eps / (2 * ms) + 1e-13)


@pytest.mark.parametrize("eps", [0.0, 1e-5])
def test_layernorm_output_zero_mean_unit_variance(eps):
    S, B, H, T, j = 16, 1, 128, 4, 3
    P, res, _, _ = _f64_case(S, B, H, T, j, 6)
    d = desc(S, B, H, T, j, oracle.F64, oracle.LAYERNORM, eps, 0.1)
    out = oracle.fwd(d, [shard_rows(x, S, B, H, T, j) for x in P], shard_rows(res, S, B, H, T, j),
                     np.ones(H), np.zeros(H))
    eps = float(np.float32(eps))  # the descriptor carries eps as fp32
    y = out["y"]
    var_h = np.var(out["h"], axis=1)
    assert np.all(np.abs(y.mean(axis=1)) <= 1e-13)
    assert np.allclose(y.var(axis=1), var_h / (var_h + eps), rtol=1e-12, atol=0)
    assert np.allclose(out["mean"], out["h"].mean(axis=1), rtol=0, atol=1e-14)


@pytest.mark.parametrize("norm", [oracle.RMSNORM, oracle.LAYERNORM])
def test_norm_matches_torch_functional_float64(norm):
    """T=1, p=0: h = residual + P_0 and y = torch's rms_norm / layer_norm of h."""
    S, B, H = 24, 2, 160
    P, res, gam, bet = _f64_case(S, B, H, 1, 0, 8, outlier=True)
    eps = 1e-6
    d = desc(S, B, H, 1, 0, oracle.F64, norm, eps, 0.0)
    out = oracle.fwd(d, [P[0].reshape(-1, H)], res.reshape(-1, H), gam,
                     bet if norm == oracle.LAYERNORM else None)
    h = torch.from_numpy(res.reshape(-1, H) + P[0].reshape(-1, H))
    assert np.array_equal(out["h"], h.numpy())
    if norm == oracle.RMSNORM:
        ref = F.rms_norm(h, (H,), weight=torch.from_numpy(gam), eps=eps)
    else:
        ref = F.layer_norm(h, (H,), torch.from_numpy(gam), torch.from_numpy(bet), eps=eps)
    assert np.allclose(out["y"], ref.numpy(), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("norm", [oracle.RMSNORM, oracle.LAYERNORM])
def test_bf16_forward_matches_exact_mode_to_one_rounding(norm):
    """The bf16 mode on bf16-representable inputs equals the exact mode up to the
    roundings it performs (fp32 sums, one bf16 rounding of h and of y)."""
    S, B, H, T, j = 16, 2, 256, 4, 2
    P, res, gam, bet = _f64_case(S, B, H, T, j, 9)
    Pb = [oracle.f32_to_bf16(x.astype(np.float32)) for x in P]
    rb = oracle.f32_to_bf16(res.astype(np.float32))
    bet = bet if norm == oracle.LAYERNORM else None
    d16 = desc(S, B, H, T, j, oracle.BF16, norm, 1e-5, 0.1)
    d64 = desc(S, B, H, T, j, oracle.F64, norm, 1e-5, 0.1)
    o16 = oracle.fwd(d16, [shard_rows(x, S, B, H, T, j) for x in Pb], shard_rows(rb, S, B, H, T, j),
                     gam, bet)
    o64 = oracle.fwd(d64, [shard_rows(oracle.bf16_to_f32(x).astype(np.float64), S, B, H, T, j)
                           for x in Pb],
                     shard_rows(oracle.bf16_to_f32(rb).astype(np.float64), S, B, H, T, j), gam, bet)
    assert np.array_equal(o16["mask"], o64["mask"])
    ulp = 2.0 ** -7  # bf16 has 8 significant bits: relative spacing <= 2^-7
    h16 = oracle.bf16_to_f32(o16["h"]).astype(np.float64)
    # fp32 intermediates: within one bf16 rounding plus fp32 noise of the exact h
    assert np.all(np.abs(h16 - o64["h"]) <= ulp * np.abs(o64["h"]) + 1e-6 * (1 + np.abs(o64["h"])))
    y16 = oracle.bf16_to_f32(o16["y"]).astype(np.float64)
    scale = np.abs(o64["y"]) + np.sqrt(np.mean(o64["y"] ** 2))
    assert np.all(np.abs(y16 - o64["y"]) <= 2 * ulp * scale)


# ---------------------------------------------------------------------------
# The fp32 activation mode (the tiny fp32 workload runs on it).

@pytest.mark.parametrize("T,p,norm", [(1, 0.0, oracle.RMSNORM), (3, 0.1, oracle.LAYERNORM),
                                      (8, 0.1, oracle.RMSNORM), (2, 0.5, oracle.LAYERNORM)])
def test_f32_forward_h_matches_torch_float32_chain(T, p, norm):
    """In the fp32 mode h is the fp32 chain P_0 + P_1 + ... (t ascending), times
    the fp32 value of 1/(1-p) where kept, plus the residual: torch's float32
    element-wise ops on the same values give the same bits."""
    S, B, H, j = 8 * T, 2, 72, T - 1
    rng = np.random.default_rng(60 + T)
    P = [(rng.standard_normal((S, B, H)) / math.sqrt(T)).astype(np.float32) for _ in range(T)]
    res = rng.standard_normal((S, B, H)).astype(np.float32)
    gam = 1 + 0.02 * rng.standard_normal(H)
    bet = 0.02 * rng.standard_normal(H) if norm == oracle.LAYERNORM else None
    d = desc(S, B, H, T, j, oracle.F32, norm, 1e-5, p)
    Ps = [shard_rows(x, S, B, H, T, j) for x in P]
    rs = shard_rows(res, S, B, H, T, j)
    out = oracle.fwd(d, Ps, rs, gam, bet)
    R = (S // T) * B
    mask = oracle.keep_mask(1234, p, j * R * H, R * H).reshape(R, H).astype(bool)
    assert np.array_equal(out["mask"].astype(bool), mask)
    acc = torch.from_numpy(Ps[0].copy())
    for x in Ps[1:]:
        acc = acc + torch.from_numpy(x)
    scale32 = torch.tensor(float(np.float32(1.0 / (1.0 - float(np.float32(p))))), dtype=torch.float32)
    z = torch.where(torch.from_numpy(mask), acc * scale32, torch.zeros((), dtype=torch.float32))
    h = torch.from_numpy(rs) + z
    assert h.dtype == torch.float32
    assert np.array_equal(out["h"].view(np.uint32), h.numpy().view(np.uint32))


@pytest.mark.parametrize("norm", [oracle.RMSNORM, oracle.LAYERNORM])
def test_f32_forward_norm_is_exact_mode_rounded_once(norm):
    """The fp32 mode's statistics are those of its stored h, and y is the exact
    mode's y of that h rounded once to fp32 (the exact mode fed h as its single
    partial, with p = 0 and a zero residual, reproduces h without rounding)."""
    S, B, H, T, j = 16, 2, 96, 4, 1
    P, res, gam, bet = _f64_case(S, B, H, T, j, 61)
    bet = bet if norm == oracle.LAYERNORM else None
    P32 = [x.astype(np.float32) for x in P]
    d32 = desc(S, B, H, T, j, oracle.F32, norm, 1e-6, 0.1)
    o32 = oracle.fwd(d32, [shard_rows(x, S, B, H, T, j) for x in P32],
                     shard_rows(res.astype(np.float32), S, B, H, T, j), gam, bet)
    R = (S // T) * B
    d64 = desc(S // T, B, H, 1, 0, oracle.F64, norm, 1e-6, 0.0)
    o64 = oracle.fwd(d64, [o32["h"].astype(np.float64)], np.zeros((R, H)), gam, bet)
    assert np.array_equal(o64["h"], o32["h"].astype(np.float64))
    assert np.array_equal(o32["rstd"], o64["rstd"])
    if norm == oracle.LAYERNORM:
        assert np.array_equal(o32["mean"], o64["mean"])
    assert np.array_equal(o32["y"].view(np.uint32), o64["y"].astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("norm,p", [(oracle.RMSNORM, 0.1), (oracle.LAYERNORM, 0.3)])
def test_f32_backward_is_exact_mode_rounded_once(norm, p):
    """The fp32 mode's backward on fp32 inputs: d_res is the exact mode's d_res
    rounded once; dP is that unrounded gradient times the fp32 value of
    1/(1-p), rounded once; dgamma / dbeta are the exact mode's sums."""
    S, B, H, T, j = 16, 2, 80, 2, 1
    rng = np.random.default_rng(62)
    R = (S // T) * B
    h = rng.standard_normal((R, H)).astype(np.float32)
    dY = rng.standard_normal((R, H)).astype(np.float32)
    mask = oracle.keep_mask(1234, p, j * R * H, R * H).reshape(R, H)
    hf = h.astype(np.float64)
    mean = hf.mean(axis=1).astype(np.float32).astype(np.float64) if norm == oracle.LAYERNORM else None
    cen = hf - (mean[:, None] if mean is not None else 0)
    rstd = (1 / np.sqrt((cen ** 2).mean(axis=1) + 1e-6)).astype(np.float32).astype(np.float64)
    gam = 1 + 0.02 * rng.standard_normal(H)
    g32 = oracle.bwd(desc(S, B, H, T, j, oracle.F32, norm, 1e-6, p), dY, h, mask, mean, rstd, gam)
    g64 = oracle.bwd(desc(S, B, H, T, j, oracle.F64, norm, 1e-6, p), dY.astype(np.float64), hf, mask,
                     mean, rstd, gam)
    assert np.array_equal(g32["d_res"].view(np.uint32), g64["d_res"].astype(np.float32).view(np.uint32))
    scale32 = np.float64(np.float32(1.0 / (1.0 - float(np.float32(p)))))
    want_dP = np.where(mask == 1, g64["d_res"] * scale32, 0.0).astype(np.float32)
    assert np.array_equal(g32["dP"].view(np.uint32), want_dP.view(np.uint32))
    assert np.array_equal(g32["dgamma"], g64["dgamma"])
    if norm == oracle.LAYERNORM:
        assert np.array_equal(g32["dbeta"], g64["dbeta"])


def test_dropout_scale_is_inverted_like_torch():
    """Kept elements carry x/(1-p) exactly as torch's dropout; the mean is kept."""
    S, B, H, p = 64, 4, 512, 0.25
    d = desc(S, B, H, 1, 0, oracle.F64, oracle.RMSNORM, 1e-6, p)
    ones = np.ones((S * B, H))
    out = oracle.fwd(d, [ones], np.zeros((S * B, H)), np.ones(H))
    torch.manual_seed(0)
    td = F.dropout(torch.ones(S * B, H, dtype=torch.float64), p=p, training=True)
    torch_kept = np.unique(td.numpy()[td.numpy() != 0])
    kept = out["h"][out["mask"] == 1]
    assert np.all(kept == torch_kept[0]) and len(torch_kept) == 1
    assert np.all(out["h"][out["mask"] == 0] == 0)
    N = S * B * H
    assert abs(out["h"].mean() - 1.0) <= 5 * math.sqrt(p * (1 - p) / N) / (1 - p)


# ---------------------------------------------------------------------------
# Backward: finite differences, torch autograd, shard sums.

def _loss_and_grads(S, B, H, T, j, norm, p, eps, seed, with_dR):
    P, res, gam, bet = _f64_case(S, B, H, T, j, seed)
    if norm == oracle.RMSNORM:
        bet = None
    rng = np.random.default_rng(seed + 100)
    R = (S // T) * B
    dY = rng.standard_normal((R, H))
    dR = rng.standard_normal((R, H)) if with_dR else None
    d = desc(S, B, H, T, j, oracle.F64, norm, eps, p)
    Ps = [shard_rows(x, S, B, H, T, j) for x in P]
    rs = shard_rows(res, S, B, H, T, j)

    def loss(Ps_, rs_, gam_, bet_):
        o = oracle.fwd(d, Ps_, rs_, gam_, bet_)
        L = np.sum(dY * o["y"])
        if with_dR:
            L += np.sum(dR * o["h"])
        return L

    o = oracle.fwd(d, Ps, rs, gam, bet)
    g = oracle.bwd(d, dY, o["h"], o["mask"], o["mean"], o["rstd"], gam, dR=dR)
    return d, Ps, rs, gam, bet, dY, dR, o, g, loss


@pytest.mark.parametrize("norm", [oracle.RMSNORM, oracle.LAYERNORM])
@pytest.mark.parametrize("with_dR", [False, True])
def test_backward_matches_central_finite_differences(norm, with_dR):
    S, B, H, T, j = 8, 1, 16, 2, 1
    d, Ps, rs, gam, bet, dY, dR, o, g, loss = _loss_and_grads(S, B, H, T, j, norm, 0.25, 1e-5, 21,
                                                              with_dR)
    step = 1e-6

    def central(make_args, arr):
        grad = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            arr[idx] += step
            lp = loss(*make_args())
            arr[idx] -= 2 * step
            lm = loss(*make_args())
            arr[idx] += step
            grad[idx] = (lp - lm) / (2 * step)
        return grad

    Pw = [x.copy() for x in Ps]
    rw, gw = rs.copy(), gam.copy()
    bw = None if bet is None else bet.copy()
    args = lambda: (Pw, rw, gw, bw)  # noqa: E731

    def close(a, b):
        return np.max(np.abs(a - b)) <= 1e-6 * max(1.0, np.max(np.abs(b)))

    for t in range(T):
        gP = central(args, Pw[t])
        assert close(g["dP"], gP), t  # same gradient for every partial
    assert close(g["d_res"], central(args, rw))
    assert close(g["dgamma"], central(args, gw))
    if bw is not None:
        assert close(g["dbeta"], central(args, bw))
    # dropped elements get no gradient through P
    assert np.all(g["dP"][o["mask"] == 0] == 0)


@pytest.mark.parametrize("norm", [oracle.RMSNORM, oracle.LAYERNORM])
def test_backward_matches_torch_autograd_float64(norm):
    S, B, H, T, j = 16, 2, 64, 4, 2
    p, eps = 0.3, 1e-6
    d, Ps, rs, gam, bet, dY, dR, o, g, _ = _loss_and_grads(S, B, H, T, j, norm, p, eps, 33, True)
    tP = [torch.from_numpy(x).requires_grad_() for x in Ps]
    tr = torch.from_numpy(rs).requires_grad_()
    tg = torch.from_numpy(gam).requires_grad_()
    tb = None if bet is None else torch.from_numpy(bet).requires_grad_()
    mask = torch.from_numpy(o["mask"].astype(bool))
    ysum = tP[0]
    for x in tP[1:]:
        ysum = ysum + x
    h = tr + torch.where(mask, ysum / (1 - np.float64(np.float32(p))), torch.zeros_like(ysum))
    if norm == oracle.RMSNORM:
        y = F.rms_norm(h, (H,), weight=tg, eps=eps)
    else:
        y = F.layer_norm(h, (H,), tg, tb, eps=eps)
    L = (torch.from_numpy(dY) * y).sum() + (torch.from_numpy(dR) * h).sum()
    L.backward()
    assert np.allclose(h.detach().numpy(), o["h"], rtol=1e-13, atol=1e-13)
    assert np.allclose(y.detach().numpy(), o["y"], rtol=1e-12, atol=1e-12)
    for t in range(T):
        assert np.allclose(tP[t].grad.numpy(), g["dP"], rtol=1e-11, atol=1e-11)
    assert np.allclose(tr.grad.numpy(), g["d_res"], rtol=1e-11, atol=1e-11)
    assert np.allclose(tg.grad.numpy(), g["dgamma"], rtol=1e-11, atol=1e-11)
    if tb is not None:
        assert np.allclose(tb.grad.numpy(), g["dbeta"], rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("norm", [oracle.RMSNORM, oracle.LAYERNORM])
def test_shard_dgamma_partials_sum_to_full_sequence_grad(norm):
    """Norm weights are replicated, so each shard's dgamma is a partial and the
    partials over all shards sum to the unsharded gradient."""
    S, B, H, T = 32, 2, 48, 4
    P, res, gam, bet = _f64_case(S, B, H, T, 0, 44)
    if norm == oracle.RMSNORM:
        bet = None
    rng = np.random.default_rng(45)
    dY = rng.standard_normal((S, B, H))
    # unsharded run: one partial holding the same sums
    Psum = P[0].copy()
    for x in P[1:]:
        Psum = Psum + x
    d1 = desc(S, B, H, 1, 0, oracle.F64, norm, 1e-6, 0.2)
    o1 = oracle.fwd(d1, [Psum.reshape(-1, H)], res.reshape(-1, H), gam, bet)
    g1 = oracle.bwd(d1, dY.reshape(-1, H), o1["h"], o1["mask"], o1["mean"], o1["rstd"], gam)
    dg = np.zeros(H)
    db = np.zeros(H)
    for j in range(T):
        d = desc(S, B, H, T, j, oracle.F64, norm, 1e-6, 0.2)
        o = oracle.fwd(d, [shard_rows(x, S, B, H, T, j) for x in P], shard_rows(res, S, B, H, T, j),
                       gam, bet)
        g = oracle.bwd(d, shard_rows(dY, S, B, H, T, j), o["h"], o["mask"], o["mean"], o["rstd"],
                       gam)
        dg += g["dgamma"]
        if bet is not None:
            db += g["dbeta"]
    assert np.allclose(dg, g1["dgamma"], rtol=1e-11, atol=1e-11)
    if bet is not None:
        assert np.allclose(db, g1["dbeta"], rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("norm", [oracle.RMSNORM, oracle.LAYERNORM])
def test_bf16_backward_matches_exact_mode_to_one_rounding(norm):
    S, B, H, T, j = 16, 2, 128, 2, 0
    rng = np.random.default_rng(55)
    R = (S // T) * B
    h = oracle.f32_to_bf16(rng.standard_normal((R, H)).astype(np.float32))
    dY = oracle.f32_to_bf16(rng.standard_normal((R, H)).astype(np.float32))
    mask = oracle.keep_mask(1234, 0.1, j * R * H, R * H).reshape(R, H)
    hf = oracle.bf16_to_f32(h).astype(np.float64)
    mean = hf.mean(axis=1).astype(np.float32).astype(np.float64) if norm == oracle.LAYERNORM else None
    cen = hf - (mean[:, None] if mean is not None else 0)
    var = (cen ** 2).mean(axis=1)
    rstd = (1 / np.sqrt(var + 1e-5)).astype(np.float32).astype(np.float64)
    gam = 1 + 0.02 * rng.standard_normal(H)
    d16 = desc(S, B, H, T, j, oracle.BF16, norm, 1e-5, 0.1)
    d64 = desc(S, B, H, T, j, oracle.F64, norm, 1e-5, 0.1)
    g16 = oracle.bwd(d16, dY, h, mask, mean, rstd, gam)
    g64 = oracle.bwd(d64, oracle.bf16_to_f32(dY).astype(np.float64), hf, mask, mean, rstd, gam)
    ulp = 2.0 ** -7
    for k in ("d_res", "dP"):
        a = oracle.bf16_to_f32(g16[k]).astype(np.float64)
        # the exact mode scales dP by 1/(1-p) in fp64, the bf16 mode by its fp32 value
        assert np.all(np.abs(a - g64[k]) <= ulp * np.abs(g64[k]) + 1e-7 * np.abs(g64[k]).max()), k
    assert np.array_equal(g16["dgamma"], g64["dgamma"])


# ---------------------------------------------------------------------------
# The pages' byte accounting (F and the memory-delta estimates).

def _golden_accounting():
    vals = {}
    with open(os.path.join(GOLDEN, "memory_accounting.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, *v = line.split()
                vals[k] = [float(x) for x in v]
    return vals


def test_memory_accounting_matches_pages():
    g = _golden_accounting()
    MiB = 1 << 20
    S, H = 2048, 768
    F2 = 2 * S * 2 * H            # bytes of one full-sequence bf16 tensor, B=2
    F4 = 2 * S * 4 * H
    assert F2 == g["F_bytes_B2_S2048_H768"][0]
    assert F2 / MiB == g["F_MiB_B2_S2048_H768"][0]
    assert F4 / MiB == g["F_MiB_B4_S2048_H768"][0]
    T = g["T"][0]
    block = 8 * F2 * (1 - 1 / T) - 3 * F2
    final = 4 * F2 * (1 - 1 / T)
    assert block / MiB == g["block_delta_MiB"][0]
    assert final / MiB == g["final_norm_delta_MiB"][0]
    est = [L * block / MiB + final / MiB for L in g["estimate_6L_plus_12_layers"]]
    assert est == g["estimate_6L_plus_12_MiB"]
    # measured deltas sit within 2 MiB of the estimates
    assert all(abs(a - b) <= 2.0 for a, b in zip(est, g["measured_delta_MiB"]))
    basic = 5 * F4 / MiB
    recompute = 2 * (F4 / 2) / MiB
    assert basic == g["recompute_basic_per_block_MiB"][0]
    assert recompute == g["recompute_per_block_MiB"][0]
    assert [L * (basic - recompute) for L in g["estimate_48L_layers"]] == g["estimate_48L_MiB"]
