"""The backward entry point that allocates nothing, through the C ABI (GPU).

sp_region_bwd_noalloc runs the same kernels as sp_region_bwd on a static
per-GPU scratch array instead of a caller's workspace, so its outputs must be
bit-identical to sp_region_bwd's on the same inputs -- call after call, with the
scratch keeping whatever the previous call left in it.
"""
import pytest
import torch

import transformer_sequence_activation_amd as sp
from transformer_sequence_activation_amd import workloads as W

pytestmark = pytest.mark.gpu

# a partial-row shard (its workspace: 4096 + 256 partial rows of 1024 floats),
# then a smaller shard on 8 column segments (4096 + 8 segment rows of 768)
ROWS = W.Workload("noalloc_rows_T2_S16384_B1_H1024", 950, 2, 16384, 1, 1024, "bf16", "rms", 1e-6, 0.1, (1,))
SEGS = W.Workload("noalloc_segs_T2_S2048_B2_H768", 951, 2, 2048, 2, 768, "bf16", "ln", 1e-5, 0.1, (0,))


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(hip_lib):
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")


def _inputs(w):
    j = w.shards[0]
    d = sp.make_desc(w.S, w.B, w.H, w.T, j, w.dtype, w.norm, w.eps, w.p, w.seed)
    P = [W.partial(w, t, "cuda") for t in range(w.T)]
    f = sp.forward(d, P, W.shard(W.residual(w, "cuda"), w, j), W.gamma(w, "cuda"),
                   W.beta(w, "cuda") if w.norm == "ln" else None)
    return d, W.shard(W.grad_y(w, "cuda"), w, j), f, W.gamma(w, "cuda")


def _outputs(d, like):
    R, H = d.R, d.H
    return {"d_res": torch.full((R, H), 7.0, dtype=like.dtype, device="cuda"),
            "dP": torch.full((R, H), 7.0, dtype=like.dtype, device="cuda"),
            "dgamma": torch.full((H,), 7.0, device="cuda"),
            "dbeta": torch.full((H,), 7.0, device="cuda") if d.norm == sp.SP_LAYERNORM else None}


def _reference(d, dY, f, gam):
    ws_bytes = sp.sp_region_bwd_workspace_size(d)
    ws = torch.zeros(max(16, ws_bytes), dtype=torch.uint8, device="cuda")
    o = _outputs(d, dY)
    rc = sp.sp_region_bwd(d, dY, f["h"], f["mask"], f["mean"], f["rstd"], gam, None, o["d_res"], o["dP"],
                          o["dgamma"], o["dbeta"], ws, ws.numel())
    assert rc == 0, sp.sp_region_strerror(rc)
    return o


def _noalloc(d, dY, f, gam):
    o = _outputs(d, dY)
    rc = sp.sp_region_bwd_noalloc(d, dY, f["h"], f["mask"], f["mean"], f["rstd"], gam, None, o["d_res"],
                                  o["dP"], o["dgamma"], o["dbeta"])
    assert rc == 0, sp.sp_region_strerror(rc)
    return o


def test_noalloc_matches_workspace_entry_point_call_after_call():
    cases = []
    for w in (ROWS, SEGS):
        d, dY, f, gam = _inputs(w)
        assert 0 < sp.sp_region_bwd_workspace_size(d) <= sp.SP_NOALLOC_SCRATCH_BYTES
        cases.append((w, d, dY, f, gam))
    assert sp.sp_region_bwd_schedule(cases[0][1]) == 0       # partial rows + finish kernel
    assert sp.sp_region_bwd_schedule(cases[1][1]) == 8       # 8 column segments
    assert cases[1][1].R * cases[1][1].H < cases[0][1].R * cases[0][1].H  # the second input is smaller
    # the larger shard, then the smaller one, then the larger one again: each
    # call starts from whatever the previous call left in the scratch
    for w, d, dY, f, gam in cases + cases[:1]:
        print(f"\n[case] {w.name}: sp_region_bwd_noalloc vs sp_region_bwd", flush=True)
        ref = _reference(d, dY, f, gam)
        got = _noalloc(d, dY, f, gam)
        torch.cuda.synchronize()
        for k in ("d_res", "dP", "dgamma", "dbeta"):
            if ref[k] is None:
                assert got[k] is None
                continue
            assert torch.equal(ref[k], got[k]), (w.name, k)
        assert bool(torch.isfinite(got["dgamma"]).all())
