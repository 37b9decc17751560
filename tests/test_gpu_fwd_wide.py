"""GPU parity of the wide forward variants (P-blocks of 64 value columns, 1024
threads: the ones the full-size SSD workloads run) at small sizes, against the
fp64 oracle.

Small problems normally take narrow P-blocks, so these tests force the P-block
(SSM_FWD_PB).  Outputs, final state and the saved boundary states (through the
reverse pass) are checked with an initial state, ragged last chunks, length 1,
head groups and sequence segments, and the wide and narrow variants agree.

Tolerances as everywhere: rel-L2 1e-4 (fp32 path), 1e-2 (bf16 path).
"""
import numpy as np
import pytest
import torch

import oracle
import selective_diagonal_ssm_amd as ssm
import workloads
from gpu_util import rel_l2, tol

pytestmark = pytest.mark.gpu

CASES = {
    # (workload, overrides, forced P-block)
    "bf16_n128": ("ssd_siso", dict(batch=2, seqlen=300, nheads=2, ngroups=2), 64),
    "bf16_n64": ("ssd_siso", dict(batch=2, seqlen=150, nheads=2, ngroups=2, dstate=64,
                                  n_real=64), 64),
    "bf16_mimo": ("ssd_mimo", dict(batch=2, seqlen=100, nheads=2, ngroups=2), 64),
    "bf16_groups": ("ssd_siso", dict(batch=1, seqlen=70, nheads=4, ngroups=2), 64),
    "bf16_len1": ("ssd_siso", dict(batch=2, seqlen=1, nheads=2, ngroups=2), 64),
}


def _np(v):
    return v.float().cpu().numpy().astype(np.float64)


def _run(prob, t, h0, save):
    y, saved, hf = ssm.forward(prob["desc"], prob["dtype"], t["x"], t["B"], t["C"], t["dt"],
                               t["A"], D=t.get("D"), save_for_backward=save, h0=h0,
                               return_final_state=True)
    torch.cuda.synchronize()
    return y, saved, hf


@pytest.mark.parametrize("nseg", [1, 3])
@pytest.mark.parametrize("case", sorted(CASES))
def test_wide_forward_matches_oracle(case, nseg, monkeypatch):
    name, kw, pb = CASES[case]
    monkeypatch.setenv("SSM_FWD_PB", str(pb))
    monkeypatch.setenv("SSM_NSEG", str(nseg))
    prob = workloads.make_problem(workloads.spec(name, **kw), seed=41, with_dy=True)
    h0 = workloads.make_state(prob["desc"], seed=43)
    print(f"[fwd-wide] case={case} nseg={nseg} desc={prob['desc']}", flush=True)
    t = workloads.to_device(prob)
    y, saved, hf = _run(prob, t, torch.from_numpy(h0).cuda(), save=True)
    yr, hr = oracle.fwd(prob, h0=h0.astype(np.float64))
    ey, eh = rel_l2(_np(y), yr), rel_l2(_np(hf), hr)
    print(f"[fwd-wide] case={case} nseg={nseg} y={ey:.2e} h_final={eh:.2e}", flush=True)
    assert ey <= tol(prob) and eh <= tol(prob), (ey, eh)
    # the saved boundary states feed the reverse pass
    g = ssm.backward(prob["desc"], prob["dtype"], t["x"], t["B"], t["C"], t["dy"], t["dt"], t["A"],
                     saved, D=t.get("D"), want=("dA", "dD", "dh0"))
    torch.cuda.synchronize()
    ref = oracle.bwd(prob, prob["dy"], h0=h0.astype(np.float64))
    errs = {k: rel_l2(_np(g[k]), ref[k]) for k in ("dx", "dB", "dC", "ddt", "dh0")}
    print(f"[fwd-wide] case={case} nseg={nseg} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()),
          flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol(prob)}
    assert not bad, bad


@pytest.mark.parametrize("case", ["bf16_n128", "bf16_mimo"])
def test_wide_and_narrow_variants_agree(case, monkeypatch):
    name, kw, pb = CASES[case]
    prob = workloads.make_problem(workloads.spec(name, **kw), seed=47)
    t = workloads.to_device(prob)
    monkeypatch.setenv("SSM_FWD_PB", str(pb))
    y_w, _, hf_w = _run(prob, t, None, save=False)
    monkeypatch.setenv("SSM_FWD_PB", "16")
    y_n, _, hf_n = _run(prob, t, None, save=False)
    ey, eh = rel_l2(_np(y_w), _np(y_n)), rel_l2(_np(hf_w), _np(hf_n))
    print(f"[fwd-wide] case={case} wide vs narrow: y={ey:.2e} h_final={eh:.2e}", flush=True)
    assert ey <= tol(prob) and eh <= tol(prob), (ey, eh)


def test_wide_forward_deterministic(monkeypatch):
    monkeypatch.setenv("SSM_FWD_PB", "64")
    name, kw, _ = CASES["bf16_n128"]
    prob = workloads.make_problem(workloads.spec(name, **kw), seed=53)
    t = workloads.to_device(prob)
    y1, _, h1 = _run(prob, t, None, save=False)
    y2, _, h2 = _run(prob, t, None, save=False)
    assert torch.equal(y1, y2) and torch.equal(h1, h2)
