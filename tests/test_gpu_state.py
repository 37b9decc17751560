"""GPU parity of the state carry (initial state h0, final state, dLoss/dh0)
against the fp64 oracle, which takes h0 as the state before token 0 and returns
the state after the last token and A_0^T g_0 (its pin P9 checks that a split
run carries the state exactly).

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
    "f32_head": ("ssd_siso", dict(dtype="f32", dstate=32, n_real=32, headdim=16, batch=2,
                                  nheads=2, ngroups=2, seqlen=150)),
    "f32_head_r2": ("ssd_mimo", dict(dtype="f32", dstate=32, n_real=32, headdim=16, rank_in=2,
                                     rank_out=2, batch=2, nheads=2, ngroups=2, seqlen=90)),
    "f32_coord_plain": ("hybrid", dict(dtype="f32", two_endpoint=False, dstate=32, n_real=16,
                                       n_pairs=8, headdim=16, batch=2, nheads=2, ngroups=2,
                                       seqlen=75)),
    "f32_hybrid": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_pairs=8, headdim=16,
                                  batch=2, nheads=2, ngroups=2, seqlen=77)),
    "bf16_ssd_siso": ("ssd_siso", dict(batch=2, seqlen=200, nheads=2, ngroups=2)),
    "bf16_ssd_mimo": ("ssd_mimo", dict(batch=2, seqlen=100, nheads=2, ngroups=2)),
    "bf16_hybrid": ("hybrid", dict(batch=2, seqlen=90, nheads=2, ngroups=2)),
}


def _fwd(prob, t, h0=None, save=False):
    y, saved, hf = ssm.forward(prob["desc"], prob["dtype"], t["x"], t["B"], t["C"], t["dt"],
                               t["A"], omega=t.get("omega"), beta=t.get("beta"),
                               gamma=t.get("gamma"), D=t.get("D"), save_for_backward=save,
                               h0=h0, return_final_state=True)
    return y, saved, hf


def _np(v):
    return v.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("case", sorted(CASES))
def test_forward_with_initial_state_matches_oracle(case):
    name, kw = CASES[case]
    prob = workloads.make_problem(workloads.spec(name, **kw), seed=3)
    h0 = workloads.make_state(prob["desc"], seed=5)
    print(f"[state-fwd] case={case} desc={prob['desc']}", flush=True)
    t = workloads.to_device(prob)
    y, _, hf = _fwd(prob, t, h0=torch.from_numpy(h0).cuda())
    torch.cuda.synchronize()
    yr, hr = oracle.fwd(prob, h0=h0.astype(np.float64))
    ey, eh = rel_l2(_np(y), yr), rel_l2(_np(hf), hr)
    print(f"[state-fwd] case={case} y={ey:.2e} h_final={eh:.2e}", flush=True)
    assert ey <= tol(prob) and eh <= tol(prob), (ey, eh)


@pytest.mark.parametrize("case", ["f32_head", "f32_head_r2", "f32_coord_plain", "bf16_ssd_siso",
                                  "bf16_ssd_mimo"])
def test_split_run_carries_state(case):
    """Two GPU runs chained through h_final -> h0 reproduce one run over the whole
    sequence (writes without a two-endpoint term, whose token-0 part is not
    carried)."""
    name, kw = CASES[case]
    prob = workloads.make_problem(workloads.spec(name, **kw), seed=7)
    L = prob["desc"]["seqlen"]
    L1 = L // 2 + 5  # not a chunk multiple
    print(f"[state-split] case={case} L={L} L1={L1}", flush=True)
    t = workloads.to_device(prob)
    y_full, _, h_full = _fwd(prob, t)

    def part(lo, hi):
        q = dict(prob)
        q["desc"] = dict(prob["desc"], seqlen=hi - lo)
        tq = {k: (v[:, lo:hi].contiguous() if k in ("x", "B", "C", "dt") else v)
              for k, v in t.items()}
        return q, tq

    q1, t1 = part(0, L1)
    y1, _, h1 = _fwd(q1, t1)
    q2, t2 = part(L1, L)
    y2, _, h2 = _fwd(q2, t2, h0=h1)
    torch.cuda.synchronize()
    ey = rel_l2(np.concatenate([_np(y1), _np(y2)], axis=1), _np(y_full))
    eh = rel_l2(_np(h2), _np(h_full))
    print(f"[state-split] case={case} y={ey:.2e} h={eh:.2e}", flush=True)
    assert ey <= tol(prob) and eh <= tol(prob), (ey, eh)


GRADS = ["dx", "dB", "dC", "ddt", "dA", "domega", "dbeta", "dgamma", "dD", "dh0"]


@pytest.mark.parametrize("case", sorted(CASES))
def test_backward_with_initial_state_matches_oracle(case):
    name, kw = CASES[case]
    prob = workloads.make_problem(workloads.spec(name, **kw), seed=11, with_dy=True)
    h0 = workloads.make_state(prob["desc"], seed=13)
    print(f"[state-bwd] case={case} desc={prob['desc']}", flush=True)
    t = workloads.to_device(prob)
    _, saved, _ = _fwd(prob, t, h0=torch.from_numpy(h0).cuda(), save=True)
    g = ssm.backward(prob["desc"], prob["dtype"], t["x"], t["B"], t["C"], t["dy"], t["dt"],
                     t["A"], saved, omega=t.get("omega"), beta=t.get("beta"),
                     gamma=t.get("gamma"), D=t.get("D"),
                     want=("dA", "domega", "dbeta", "dgamma", "dD", "dh0"))
    torch.cuda.synchronize()
    ref = oracle.bwd(prob, prob["dy"], h0=h0.astype(np.float64))
    errs = {k: rel_l2(_np(g[k]), ref[k]) for k in GRADS if k in g and ref.get(k) is not None}
    print(f"[state-bwd] case={case} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()),
          flush=True)
    assert "dh0" in errs
    bad = {k: v for k, v in errs.items() if not v <= tol(prob)}
    assert not bad, bad


SEG_CASES = {
    "f32_head": ("ssd_siso", dict(dtype="f32", dstate=32, n_real=32, headdim=16, batch=1,
                                  nheads=2, ngroups=2, seqlen=700)),
    "f32_hybrid": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_pairs=8, headdim=16,
                                  batch=1, nheads=2, ngroups=2, seqlen=333)),
    "bf16_ssd_mimo": ("ssd_mimo", dict(batch=1, seqlen=700, nheads=2, ngroups=2)),
    "bf16_hybrid": ("hybrid", dict(batch=1, seqlen=500, nheads=2, ngroups=2)),
}


@pytest.mark.parametrize("nseg", [1, 3, 7])
@pytest.mark.parametrize("case", sorted(SEG_CASES))
def test_sequence_segments_match_oracle(case, nseg, monkeypatch):
    """The forward split into sequence segments (local pass, combine, full pass)
    gives the oracle's outputs, final state and saved boundary states, with an
    initial state."""
    monkeypatch.setenv("SSM_NSEG", str(nseg))
    name, kw = SEG_CASES[case]
    prob = workloads.make_problem(workloads.spec(name, **kw), seed=17)
    h0 = workloads.make_state(prob["desc"], seed=19)
    print(f"[segments] case={case} nseg={nseg} desc={prob['desc']}", flush=True)
    t = workloads.to_device(prob)
    y, saved, hf = _fwd(prob, t, h0=torch.from_numpy(h0).cuda(), save=True)
    torch.cuda.synchronize()
    yr, hr = oracle.fwd(prob, h0=h0.astype(np.float64))
    ey, eh = rel_l2(_np(y), yr), rel_l2(_np(hf), hr)
    print(f"[segments] case={case} nseg={nseg} y={ey:.2e} h_final={eh:.2e}", flush=True)
    assert ey <= tol(prob) and eh <= tol(prob), (ey, eh)
    # the gradients read the saved boundary states: check them through the backward
    if name != "ssd_siso" or prob["dtype"] == "f32":
        pd = workloads.make_problem(workloads.spec(name, **kw), seed=17, with_dy=True)
        td = workloads.to_device(pd)
        g = ssm.backward(pd["desc"], pd["dtype"], td["x"], td["B"], td["C"], td["dy"], td["dt"],
                         td["A"], saved, omega=td.get("omega"), beta=td.get("beta"),
                         gamma=td.get("gamma"), D=td.get("D"), want=("dA", "dD", "dh0"))
        torch.cuda.synchronize()
        ref = oracle.bwd(pd, pd["dy"], h0=h0.astype(np.float64))
        errs = {k: rel_l2(_np(g[k]), ref[k]) for k in ("dx", "dC", "ddt", "dh0")}
        print(f"[segments] case={case} nseg={nseg} " +
              " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
        bad = {k: v for k, v in errs.items() if not v <= tol(pd)}
        assert not bad, bad


# two-endpoint forwards without saved states walk two chunks per step; segment
# boundaries at an even number of chunks (16 tokens each) keep that path
DOUBLE_CASES = {
    "f32_hybrid": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_pairs=8, headdim=16,
                                  batch=1, nheads=2, ngroups=2, seqlen=501)),
    "bf16_hybrid": ("hybrid", dict(batch=1, seqlen=501, nheads=2, ngroups=2)),
    "bf16_hybrid_r1": ("hybrid_r1", dict(batch=1, seqlen=250, nheads=2, ngroups=2)),
}


@pytest.mark.parametrize("nseg", [1, 2, 4])
@pytest.mark.parametrize("case", sorted(DOUBLE_CASES))
def test_double_chunk_forward_matches_oracle(case, nseg, monkeypatch):
    """The two-chunk forward (no saved states) with h0 and sequence segments gives the
    oracle's outputs and final state, and agrees with the one-chunk walk."""
    monkeypatch.setenv("SSM_NSEG", str(nseg))
    name, kw = DOUBLE_CASES[case]
    prob = workloads.make_problem(workloads.spec(name, **kw), seed=23)
    h0 = workloads.make_state(prob["desc"], seed=29)
    print(f"[double] case={case} nseg={nseg} desc={prob['desc']}", flush=True)
    t = workloads.to_device(prob)
    h0t = torch.from_numpy(h0).cuda()
    y, _, hf = _fwd(prob, t, h0=h0t)
    monkeypatch.setenv("SSM_FWD_SINGLE", "1")
    y1, _, hf1 = _fwd(prob, t, h0=h0t)
    torch.cuda.synchronize()
    yr, hr = oracle.fwd(prob, h0=h0.astype(np.float64))
    ey, eh = rel_l2(_np(y), yr), rel_l2(_np(hf), hr)
    e1, eh1 = rel_l2(_np(y), _np(y1)), rel_l2(_np(hf), _np(hf1))
    print(f"[double] case={case} nseg={nseg} y={ey:.2e} h_final={eh:.2e} vs one-chunk "
          f"y={e1:.2e} h_final={eh1:.2e}", flush=True)
    assert ey <= tol(prob) and eh <= tol(prob), (ey, eh)
    assert e1 <= tol(prob) and eh1 <= tol(prob), (e1, eh1)


@pytest.mark.parametrize("name,batch,seqlen", [("ssd_siso", 2, 0), ("hybrid", 2, 0),
                                               ("ssd_siso", 0, 64), ("hybrid", 0, 64)])
def test_empty_problem_writes_nonempty_outputs(name, batch, seqlen):
    """No tokens (or no slices): the final state is h0 (zero without it), and dA, domega,
    dD and dh0, sums over no tokens, are zero.  The outputs start as NaN, so one left
    unwritten fails."""
    from selective_diagonal_ssm_amd import _lib
    prob = workloads.make_problem(workloads.spec(name, batch=batch, seqlen=seqlen, nheads=2,
                                                 ngroups=2), seed=3, with_dy=True)
    d = prob["desc"]
    print(f"[empty] {name} batch={batch} seqlen={seqlen}", flush=True)
    t = workloads.to_device(prob)
    desc = _lib.make_desc(d, prob["dtype"])
    dev = t["dt"].device
    shape = (batch, d["nheads"], d["dstate"], d["headdim"])
    nan = float("nan")
    h0 = torch.randn(shape, dtype=torch.float32, device=dev)
    y = torch.empty((batch, seqlen, d["nheads"], d["rank_out"], d["headdim"]),
                    dtype=t["x"].dtype, device=dev)
    for init in (h0, None):
        hf = torch.full(shape, nan, dtype=torch.float32, device=dev)
        _lib.scan_fwd(desc, t["x"], t["B"], t["C"], t["dt"], t["A"], y, omega=t.get("omega"),
                      beta=t.get("beta"), gamma=t.get("gamma"), D=t.get("D"), h0=init,
                      h_final=hf)
        torch.cuda.synchronize()
        assert torch.equal(hf, h0 if init is not None else torch.zeros_like(hf))

    g = {"dA": torch.full_like(t["A"], nan), "dh0": torch.full(shape, nan, device=dev)}
    if t.get("omega") is not None:
        g["domega"] = torch.full_like(t["omega"], nan)
    if t.get("D") is not None:
        g["dD"] = torch.full_like(t["D"], nan)
    te = t.get("beta") is not None
    _lib.scan_bwd(desc, t["x"], t["B"], t["C"], t["dy"], t["dt"], t["A"], None,
                  torch.empty_like(t["x"]), torch.empty_like(t["B"]), torch.empty_like(t["C"]),
                  torch.empty_like(t["dt"]), omega=t.get("omega"), beta=t.get("beta"),
                  gamma=t.get("gamma"), D=t.get("D"), dA=g["dA"], domega=g.get("domega"),
                  dbeta=torch.empty_like(t["dt"]) if te else None,
                  dgamma=torch.empty_like(t["dt"]) if te else None, dD=g.get("dD"),
                  dh0=g["dh0"])
    torch.cuda.synchronize()
    for k, v in g.items():
        assert torch.count_nonzero(v).item() == 0, k
