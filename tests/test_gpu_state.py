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
    "f32_hybrid_pair_rates": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_pairs=8,
                                             headdim=16, batch=2, nheads=2, ngroups=2,
                                             seqlen=77, pair_rate_per_pair=True)),
    "bf16_hybrid_pair_rates": ("hybrid", dict(batch=2, seqlen=90, nheads=2, ngroups=2,
                                              pair_rate_per_pair=True)),
    # real static rows next to dynamic rows and pairs
    "f32_hybrid_static": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_static=8,
                                         n_pairs=8, headdim=16, batch=2, nheads=2, ngroups=2,
                                         seqlen=77)),
    "bf16_hm75_static": ("hybrid", dict(batch=2, seqlen=90, nheads=2, ngroups=2, n_real=16,
                                        n_static=8, n_pairs=24)),
    # steep per-row decay (every chunk redone token by token) and a spike mix
    "f32_hybrid_steep": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_pairs=8,
                                        headdim=16, batch=2, nheads=2, ngroups=2, seqlen=77,
                                        dt_mean=2.0, A_lo=16.0, A_hi=16.0)),
    "bf16_hybrid_spikes": ("hybrid", dict(batch=2, seqlen=90, nheads=3, ngroups=3,
                                          dt_spike_prob=[0.0, 0.1, 0.5], dt_spike_mean=3.0)),
}


def _fwd(prob, t, h0=None, save=False):
    y, saved, hf = ssm.forward(prob["desc"], prob["dtype"], t["x"], t["B"], t["C"], t["dt"],
                               t["A"], omega=t.get("omega"), beta=t.get("beta"),
                               gamma=t.get("gamma"), D=t.get("D"), save_for_backward=save,
                               h0=h0, return_final_state=True, chunk=prob.get("chunk", 0))
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
    # static rows: the combines decay them by the ranges' token counts
    "f32_hybrid_static": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_static=8,
                                         n_pairs=8, headdim=16, batch=1, nheads=2, ngroups=2,
                                         seqlen=333, A_static_lo=0.001, A_static_hi=0.05)),
    "bf16_coord_plain_static": ("hybrid", dict(batch=1, seqlen=500, nheads=2, ngroups=2,
                                               two_endpoint=False, n_static=16,
                                               A_static_lo=0.001, A_static_hi=0.05)),
    # spikes in a few places only: segments with a steep chunk are redone token by token
    # from their combined incoming state, the others stay on the chunked path
    "bf16_hybrid_spikes": ("hybrid", dict(batch=1, seqlen=500, nheads=2, ngroups=2,
                                          dt_spike_prob=[0.0, 0.02], dt_spike_mean=3.0)),
    "f32_hybrid_spikes": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_pairs=8,
                                         headdim=16, batch=1, nheads=2, ngroups=2, seqlen=333,
                                         dt_spike_prob=[0.02, 0.0], dt_spike_mean=3.0)),
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
# boundaries at an even number of chunks (16 tokens each, asked for) keep that path
DOUBLE_CASES = {
    "f32_hybrid": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_pairs=8, headdim=16,
                                  batch=1, nheads=2, ngroups=2, seqlen=501, chunk=16)),
    "bf16_hybrid": ("hybrid", dict(batch=1, seqlen=501, nheads=2, ngroups=2, chunk=16)),
    "bf16_hybrid_r1": ("hybrid_r1", dict(batch=1, seqlen=250, nheads=2, ngroups=2, chunk=16)),
    "bf16_hybrid_static": ("hybrid", dict(batch=1, seqlen=501, nheads=2, ngroups=2,
                                          n_static=16, A_static_lo=0.001, A_static_hi=0.05,
                                          chunk=16)),
    "bf16_hybrid_spikes": ("hybrid", dict(batch=1, seqlen=501, nheads=2, ngroups=2,
                                          dt_spike_prob=[0.0, 0.02], dt_spike_mean=3.0,
                                          chunk=16)),
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


# ---------------------------------------------------------------- two-endpoint carry
CARRY = {
    "f32_hybrid": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_pairs=8, headdim=16,
                                  batch=2, nheads=2, ngroups=2, seqlen=77), 0),
    "bf16_hybrid": ("hybrid", dict(batch=2, seqlen=150, nheads=2, ngroups=2), 0),
    "bf16_hybrid_r1": ("hybrid_r1", dict(batch=2, seqlen=150, nheads=2, ngroups=2), 0),
    "bf16_groups": ("hybrid", dict(batch=2, seqlen=90, nheads=4, ngroups=2), 0),
    "f32_groups_segments": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_pairs=8,
                                           headdim=16, batch=1, nheads=3, ngroups=1,
                                           seqlen=333), 3),
    "bf16_segments": ("hybrid", dict(batch=1, seqlen=500, nheads=2, ngroups=2), 3),
    "bf16_static_segments": ("hybrid", dict(batch=1, seqlen=500, nheads=2, ngroups=2,
                                            n_static=8, A_static_lo=0.001, A_static_hi=0.05), 3),
    "f32_steep": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_pairs=8, headdim=16,
                                 batch=2, nheads=2, ngroups=2, seqlen=77, dt_mean=2.0,
                                 A_lo=16.0, A_hi=16.0), 0),
}


def _carry_inputs(prob, seed):
    d = prob["desc"]
    rng = np.random.default_rng(seed)
    io = torch.bfloat16 if prob["dtype"] == "bf16" else torch.float32
    sc = workloads.spec("hybrid")["xbc_scale"]
    xp = (rng.standard_normal((d["batch"], d["nheads"], d["rank_in"], d["headdim"])) * sc
          ).astype(np.float32)
    bp = (rng.standard_normal((d["batch"], d["ngroups"], d["rank_in"], d["dstate"])) * sc
          ).astype(np.float32)
    if prob["dtype"] == "bf16":
        xp, bp = workloads.round_bf16(xp), workloads.round_bf16(bp)
    h0 = workloads.make_state(d, seed=seed + 1, scale=0.5)
    dhf = workloads.make_state(d, seed=seed + 2)
    t = {"x_prev": torch.from_numpy(xp).cuda().to(io), "B_prev": torch.from_numpy(bp).cuda().to(io),
         "h0": torch.from_numpy(h0).cuda(), "dh_final": torch.from_numpy(dhf).cuda()}
    return xp, bp, h0, dhf, t


@pytest.mark.parametrize("case", sorted(CARRY))
def test_carried_token_forward_and_backward_match_oracle(case, monkeypatch):
    """The token before the sequence (x_prev, B_prev), h0 and an upstream gradient of the
    final state: y, h_final and every gradient, including dx_prev, dB_prev and dh0,
    against the oracle."""
    name, kw, nseg = CARRY[case]
    if nseg:
        monkeypatch.setenv("SSM_NSEG", str(nseg))
    prob = workloads.make_problem(workloads.spec(name, **kw), seed=31, with_dy=True)
    xp, bp, h0, dhf, c = _carry_inputs(prob, 37)
    print(f"[carry] case={case} desc={prob['desc']}", flush=True)
    t = workloads.to_device(prob)
    for save in (False, True):
        y, saved, hf = ssm.forward(prob["desc"], prob["dtype"], t["x"], t["B"], t["C"], t["dt"],
                                   t["A"], omega=t.get("omega"), beta=t.get("beta"),
                                   gamma=t.get("gamma"), D=t.get("D"), save_for_backward=save,
                                   h0=c["h0"], return_final_state=True, x_prev=c["x_prev"],
                                   B_prev=c["B_prev"])
        torch.cuda.synchronize()
        yr, hr = oracle.fwd(prob, h0=h0.astype(np.float64), x_prev=xp, B_prev=bp)
        ey, eh = rel_l2(_np(y), yr), rel_l2(_np(hf), hr)
        print(f"[carry] case={case} save={save} y={ey:.2e} h_final={eh:.2e}", flush=True)
        assert ey <= tol(prob) and eh <= tol(prob), (ey, eh)
    g = ssm.backward(prob["desc"], prob["dtype"], t["x"], t["B"], t["C"], t["dy"], t["dt"],
                     t["A"], saved, omega=t.get("omega"), beta=t.get("beta"),
                     gamma=t.get("gamma"), D=t.get("D"),
                     want=("dA", "domega", "dbeta", "dgamma", "dD", "dh0"),
                     x_prev=c["x_prev"], B_prev=c["B_prev"], dh_final=c["dh_final"])
    torch.cuda.synchronize()
    ref = oracle.bwd(prob, prob["dy"], h0=h0.astype(np.float64), x_prev=xp, B_prev=bp,
                     dh_final=dhf.astype(np.float64))
    errs = {k: rel_l2(_np(g[k]), ref[k]) for k in GRADS + ["dx_prev", "dB_prev"]
            if k in g and ref.get(k) is not None}
    print(f"[carry] case={case} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert {"dh0", "dx_prev", "dB_prev", "dbeta"} <= set(errs)
    bad = {k: v for k, v in errs.items() if not v <= tol(prob)}
    assert not bad, bad


@pytest.mark.parametrize("case", ["f32_hybrid", "bf16_hybrid", "bf16_hybrid_r1"])
def test_two_endpoint_split_run_chains_through_the_carry(case):
    """Two GPU calls over the halves of a two-endpoint sequence, the second continued with
    the first one's h_final and last token, give one run's outputs; their backward passes
    chained (the second's dh0 as the first's dh_final, its dx_prev / dB_prev added to the
    first's last token) give one run's gradients."""
    name, kw, _ = CARRY[case]
    prob = workloads.make_problem(workloads.spec(name, **kw), seed=41, with_dy=True)
    L = prob["desc"]["seqlen"]
    L1 = L // 2 + 3
    t = workloads.to_device(prob)
    kw_p = dict(omega=t.get("omega"), D=t.get("D"))

    def part(lo, hi):
        return {k: (v[:, lo:hi].contiguous() if k in ("x", "B", "C", "dt", "beta", "gamma", "dy")
                    else v) for k, v in t.items()}

    def fwd(d, tq, **extra):
        return ssm.forward(d, prob["dtype"], tq["x"], tq["B"], tq["C"], tq["dt"], tq["A"],
                           beta=tq["beta"], gamma=tq["gamma"], save_for_backward=True,
                           return_final_state=True, **kw_p, **extra)

    def bwd(d, tq, saved, **extra):
        return ssm.backward(d, prob["dtype"], tq["x"], tq["B"], tq["C"], tq["dy"], tq["dt"],
                            tq["A"], saved, beta=tq["beta"], gamma=tq["gamma"],
                            want=("dA", "domega", "dbeta", "dgamma", "dD", "dh0"), **kw_p, **extra)

    d1, d2 = dict(prob["desc"], seqlen=L1), dict(prob["desc"], seqlen=L - L1)
    t1, t2 = part(0, L1), part(L1, L)
    y, sv, hf = fwd(prob["desc"], t)
    g = bwd(prob["desc"], t, sv)
    carry = dict(x_prev=t["x"][:, L1 - 1].contiguous(), B_prev=t["B"][:, L1 - 1].contiguous())
    y1, s1, h1 = fwd(d1, t1)
    y2, s2, h2 = fwd(d2, t2, h0=h1, **carry)
    g2 = bwd(d2, t2, s2, **carry)
    g1 = bwd(d1, t1, s1, dh_final=g2["dh0"])
    torch.cuda.synchronize()
    tl = tol(prob)
    assert rel_l2(_np(torch.cat([y1, y2], 1)), _np(y)) <= tl
    assert rel_l2(_np(h2), _np(hf)) <= tl
    dx1, dB1 = g1["dx"].float().clone(), g1["dB"].float().clone()
    dx1[:, L1 - 1] += g2["dx_prev"].float()
    dB1[:, L1 - 1] += g2["dB_prev"].float()
    errs = {"dx": rel_l2(_np(torch.cat([dx1, g2["dx"].float()], 1)), _np(g["dx"])),
            "dB": rel_l2(_np(torch.cat([dB1, g2["dB"].float()], 1)), _np(g["dB"]))}
    for k in ("dC", "ddt", "dbeta", "dgamma"):
        errs[k] = rel_l2(_np(torch.cat([g1[k], g2[k]], 1)), _np(g[k]))
    for k in ("dA", "domega", "dD"):
        errs[k] = rel_l2(_np(g1[k] + g2[k]), _np(g[k]))
    errs["dh0"] = rel_l2(_np(g1["dh0"]), _np(g["dh0"]))
    print(f"[carry-chain] case={case} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()),
          flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tl}
    assert not bad, bad


def _prefix(prob, n):
    """The problem cut to its first n tokens."""
    out = dict(prob)
    out["desc"] = dict(prob["desc"], seqlen=n)
    for k in ("x", "B", "C", "dt", "beta", "gamma", "dy"):
        if prob.get(k) is not None:
            out[k] = np.ascontiguousarray(prob[k][:, :n])
    return out


def _saved_states(prob, saved, q):
    """The saved chunk-boundary states as [batch][nheads][slots][N][P] float64."""
    d = prob["desc"]
    slots = (d["seqlen"] + q - 1) // q + 1
    shape = (d["batch"], d["nheads"], slots, d["dstate"], d["headdim"])
    flat = saved.view(torch.bfloat16) if prob["dtype"] == "bf16" else saved
    return _np(flat[: int(np.prod(shape))].reshape(shape))


# ragged ends of the double-chunk walk: a last 32-token chunk of exactly 16 tokens (no middle
# state of its own: its end is the last 16-token slot), of 17, and of one token
RAGGED_SAVE = {
    f"{dt}_hybrid_L{L}": ("hybrid", dict(DOUBLE_CASES[f"{dt}_hybrid"][1], seqlen=L))
    for dt in ("bf16", "f32") for L in (496, 497, 481)
}
# steep per-row decay (every double chunk flagged and redone token by token, which stores the
# same 16-token slots), with a ragged end of 9 tokens
RAGGED_SAVE.update({
    f"{dt}_hybrid_steep_L201": ("hybrid", dict(DOUBLE_CASES[f"{dt}_hybrid"][1], seqlen=201,
                                               dt_mean=2.0, A_lo=16.0, A_hi=16.0))
    for dt in ("bf16", "f32")
})


@pytest.mark.parametrize("nseg", [1, 4])
@pytest.mark.parametrize("case", sorted(DOUBLE_CASES) + sorted(RAGGED_SAVE))
def test_saved_states_match_oracle(case, nseg, monkeypatch):
    """Every slot of the saved chunk-boundary states (two-endpoint per-row decay at an even
    rank walks double chunks and also saves the state after each one's first half) is the
    oracle's state after that many tokens, and agrees with the one-chunk walk; y and the
    final state match the oracle."""
    monkeypatch.setenv("SSM_NSEG", str(nseg))
    name, kw = DOUBLE_CASES[case] if case in DOUBLE_CASES else RAGGED_SAVE[case]
    prob = workloads.make_problem(workloads.spec(name, **kw), seed=31)
    h0 = workloads.make_state(prob["desc"], seed=37)
    q = prob["chunk"]
    L = prob["desc"]["seqlen"]
    print(f"[saved] case={case} nseg={nseg} desc={prob['desc']}", flush=True)
    t = workloads.to_device(prob)
    h0t = torch.from_numpy(h0).cuda()
    y, saved, hf = _fwd(prob, t, h0=h0t, save=True)
    monkeypatch.setenv("SSM_FWD_SINGLE", "1")
    y1, saved1, hf1 = _fwd(prob, t, h0=h0t, save=True)
    torch.cuda.synchronize()
    yr, hr = oracle.fwd(prob, h0=h0.astype(np.float64))
    ey, eh = rel_l2(_np(y), yr), rel_l2(_np(hf), hr)
    S, S1 = _saved_states(prob, saved, q), _saved_states(prob, saved1, q)
    nslots = S.shape[2]
    e1 = rel_l2(S, S1)
    # slot k holds the state after min(k q, L) tokens: the first few (a double chunk's
    # half and end), one in the middle and the last two (a ragged end)
    errs = {}
    for k in sorted({0, 1, 2, 3, nslots // 2 | 1, nslots - 2, nslots - 1}):
        n = min(k * q, L)
        ref = h0.astype(np.float64) if n == 0 else oracle.fwd(_prefix(prob, n), h0=h0.astype(np.float64))[1]
        errs[k] = rel_l2(S[:, :, k], ref)
    print(f"[saved] case={case} nseg={nseg} y={ey:.2e} h_final={eh:.2e} slots vs one-chunk "
          f"{e1:.2e} vs oracle " + " ".join(f"{k}:{v:.2e}" for k, v in errs.items()), flush=True)
    assert ey <= tol(prob) and eh <= tol(prob), (ey, eh)
    assert e1 <= tol(prob), e1
    assert all(v <= tol(prob) for v in errs.values()), errs
