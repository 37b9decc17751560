"""The allocation-free forward entry point (ssm_scan_fwd_noalloc): its workspace is the
library's static scratch array.  Checked against ssm_scan_fwd (caller workspace) on two
calls in a row, the second smaller, and its size limit on the host."""
import ctypes

import numpy as np
import pytest

import selective_diagonal_ssm_amd as ssm
import workloads
from selective_diagonal_ssm_amd import _lib


def _desc(name, **kw):
    s = workloads.spec(name, **kw)
    return s, _lib.make_desc({k: s[k] for k in workloads.DESC_KEYS}, s["dtype"])


def test_noalloc_rejects_problems_beyond_the_scratch_array():
    """A problem whose forward workspace exceeds the array is refused with
    SSM_ERR_SCRATCH before anything touches the GPU (so this runs on a CPU-only host)."""
    _, d = _desc("hybrid_bwd", batch=4)
    assert ssm.workspace_bytes(d, False) > ssm.scratch_bytes()
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: the call stops first
    args = _lib.SsmFwdArgs(fake, fake, fake, fake, fake, fake, fake, fake, fake, fake,
                           None, None, None, None)
    rc = ssm.load().ssm_scan_fwd_noalloc(ctypes.byref(d), ctypes.byref(args), None)
    assert rc == -8, rc
    # within the limit the same descriptor family is accepted by the size check
    _, small = _desc("hybrid_bwd")
    assert ssm.workspace_bytes(small, False) <= ssm.scratch_bytes()


def _run(prob, noalloc, save, h0=None):
    import torch
    t = workloads.to_device(prob)
    d = prob["desc"]
    desc = _lib.make_desc(d, prob["dtype"])
    y = torch.empty((d["batch"], d["seqlen"], d["nheads"], d["rank_out"], d["headdim"]),
                    dtype=t["x"].dtype, device="cuda")
    saved = (torch.empty((ssm.saved_bytes(desc) + 3) // 4, dtype=torch.float32, device="cuda")
             if save else None)
    hf = torch.empty((d["batch"], d["nheads"], d["dstate"], d["headdim"]), dtype=torch.float32,
                     device="cuda")
    kw = dict(omega=t.get("omega"), beta=t.get("beta"), gamma=t.get("gamma"), D=t.get("D"),
              saved=saved, h0=h0, h_final=hf)
    if noalloc:
        _lib.scan_fwd_noalloc(desc, t["x"], t["B"], t["C"], t["dt"], t["A"], y, **kw)
    else:
        wsb = ssm.workspace_bytes(desc, False)
        assert wsb > 0  # the case exercises the workspace (sequence segments)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        _lib.scan_fwd(desc, t["x"], t["B"], t["C"], t["dt"], t["A"], y, ws=ws, **kw)
    torch.cuda.synchronize()
    return y, saved, hf


@pytest.mark.gpu
@pytest.mark.parametrize("name,kw1,kw2", [
    ("hybrid", dict(batch=1, seqlen=2048, nheads=2, ngroups=2),
     dict(batch=1, seqlen=700, nheads=1, ngroups=1)),
    ("ssd_mimo", dict(batch=1, seqlen=3000, nheads=2, ngroups=2),
     dict(batch=1, seqlen=900, nheads=1, ngroups=1)),
    ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_pairs=8, headdim=16, batch=1,
                    seqlen=1500, nheads=2, ngroups=2),
     dict(dtype="f32", dstate=32, n_real=16, n_pairs=8, headdim=16, batch=1, seqlen=500,
          nheads=1, ngroups=1)),
])
def test_noalloc_matches_caller_workspace_twice(name, kw1, kw2):
    """Two calls in a row, the second on a smaller problem (the array keeps the first
    call's contents): y, the saved chunk states and h_final equal those of ssm_scan_fwd
    with a caller workspace, and y is within the parity tolerance of the oracle."""
    import torch

    import oracle
    from gpu_util import rel_l2, tol
    for seed, kw in ((0, kw1), (1, kw2)):
        prob = workloads.make_problem(workloads.spec(name, **kw), seed=seed)
        h0 = torch.from_numpy(workloads.make_state(prob["desc"], seed=seed + 5)).cuda()
        print(f"[noalloc] {name} {kw}", flush=True)
        ya, sa, ha = _run(prob, noalloc=False, save=True, h0=h0)
        yb, sb, hb = _run(prob, noalloc=True, save=True, h0=h0)
        yc, _, _ = _run(prob, noalloc=True, save=False)
        assert torch.equal(ya, yb) and torch.equal(sa, sb) and torch.equal(ha, hb)
        ref, _ = oracle.fwd(prob)
        err = rel_l2(yc.float().cpu().numpy(), ref)
        print(f"[noalloc] {name} rel_l2={err:.2e}", flush=True)
        assert err <= tol(prob), err
        assert np.isfinite(yb.float().cpu().numpy()).all()
