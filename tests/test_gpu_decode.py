"""GPU parity of the single-token recurrent step (ssm_decode_step) against the
fp64 oracle's sequential recurrence.

A run of T steps from a seeded state h0 must reproduce the oracle's outputs
y_0..y_{T-1} token by token and its final state (the step passes the previous
token's x and B for the two-endpoint write, the first step none, exactly as the
recurrence has B_{-1} X_{-1} = 0).  A prefill with the chunked scan followed by
steps must reproduce the oracle over the whole sequence.

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
    "f32_siso": ("siso_f32", dict(batch=2, nheads=3, ngroups=3)),
    "f32_head_r2": ("ssd_mimo", dict(dtype="f32", dstate=32, n_real=32, headdim=16, rank_in=2,
                                     rank_out=2, batch=2, nheads=2, ngroups=2)),
    "f32_r2_o3": ("ssd_mimo", dict(dtype="f32", dstate=32, n_real=32, headdim=32, rank_in=2,
                                   rank_out=3, has_D=False, batch=2, nheads=4, ngroups=2)),
    "f32_coord_plain": ("hybrid", dict(dtype="f32", two_endpoint=False, dstate=32, n_real=16,
                                       n_pairs=8, headdim=16, batch=2, nheads=2, ngroups=2)),
    "f32_hybrid": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_pairs=8, headdim=48,
                                  batch=2, nheads=2, ngroups=1)),
    "f32_pairs_only": ("hybrid", dict(dtype="f32", dstate=16, n_real=0, n_pairs=8, headdim=16,
                                      batch=1, nheads=2, ngroups=2)),
    "bf16_ssd_siso": ("ssd_siso", dict(batch=2, nheads=3, ngroups=3)),
    "bf16_ssd_mimo": ("ssd_mimo", dict(batch=2, nheads=2, ngroups=2)),
    "bf16_hybrid": ("hybrid", dict(batch=2, nheads=2, ngroups=2)),
    "bf16_p256": ("ssd_siso", dict(batch=1, nheads=2, ngroups=2, headdim=256, dstate=64,
                                   n_real=64)),
    # one decay rate per (head, pair); steps given directly (no softplus)
    "f32_hybrid_pair_rates": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_pairs=8,
                                             headdim=16, batch=2, nheads=2, ngroups=2,
                                             pair_rate_per_pair=True)),
    "bf16_hybrid_pair_rates": ("hybrid", dict(batch=2, nheads=2, ngroups=2,
                                              pair_rate_per_pair=True)),
    "f32_hybrid_no_softplus": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_pairs=8,
                                              headdim=16, batch=2, nheads=2, ngroups=2,
                                              dt_softplus=False, dt_mean=0.1, dt_std=0.02)),
    # real static rows (decay e^{-A} per token whatever the step) next to dynamic rows and pairs
    "f32_hybrid_static": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_static=8,
                                         n_pairs=8, headdim=16, batch=2, nheads=2, ngroups=2)),
    "bf16_hm75_static": ("hybrid", dict(batch=2, nheads=2, ngroups=2, n_real=16, n_static=8,
                                        n_pairs=24)),
}


def _np(v):
    return v.float().cpu().numpy().astype(np.float64)


def _steps(prob, t, state, lo, hi):
    """Run tokens lo..hi-1 through the step kernel; returns the stacked y."""
    ys = []
    for s in range(lo, hi):
        prev = s > 0 and prob["desc"]["two_endpoint"]
        y = ssm.decode_step(prob["desc"], prob["dtype"], t["x"][:, s].contiguous(),
                            t["B"][:, s].contiguous(), t["C"][:, s].contiguous(),
                            t["dt"][:, s].contiguous(), t["A"], state, omega=t.get("omega"),
                            beta=None if t.get("beta") is None else t["beta"][:, s].contiguous(),
                            gamma=None if t.get("gamma") is None else t["gamma"][:, s].contiguous(),
                            D=t.get("D"),
                            x_prev=t["x"][:, s - 1].contiguous() if prev else None,
                            B_prev=t["B"][:, s - 1].contiguous() if prev else None)
        ys.append(y)
    torch.cuda.synchronize()
    return np.stack([_np(y) for y in ys], axis=1)


@pytest.mark.parametrize("case", sorted(CASES))
def test_decode_steps_match_oracle(case):
    name, kw = CASES[case]
    T = 7
    prob = workloads.make_problem(workloads.spec(name, seqlen=T, **kw), seed=11)
    h0 = workloads.make_state(prob["desc"], seed=13, scale=0.5)
    print(f"[decode] case={case} desc={prob['desc']}", flush=True)
    t = workloads.to_device(prob)
    state = torch.from_numpy(h0).cuda()
    y = _steps(prob, t, state, 0, T)
    yr, hr = oracle.fwd(prob, h0=h0.astype(np.float64))
    ey, eh = rel_l2(y, yr), rel_l2(_np(state), hr)
    ey0 = rel_l2(y[:, :1], yr[:, :1])
    print(f"[decode] case={case} y={ey:.2e} y0={ey0:.2e} state={eh:.2e}", flush=True)
    assert ey <= tol(prob) and ey0 <= tol(prob) and eh <= tol(prob), (ey, ey0, eh)


@pytest.mark.parametrize("case", ["f32_siso", "f32_head_r2", "f32_coord_plain", "f32_hybrid",
                                  "bf16_ssd_siso", "bf16_hybrid"])
def test_prefill_then_decode_matches_oracle(case):
    """The scan over the first L1 tokens hands its final state to the step kernel,
    which continues the sequence (with the previous token's x and B for the
    two-endpoint write, so the continuation is exact in every mode)."""
    name, kw = CASES[case]
    L, L1 = 40, 33
    prob = workloads.make_problem(workloads.spec(name, seqlen=L, **kw), seed=17)
    if prob["desc"]["rank_in"] != prob["desc"]["rank_out"]:
        pytest.skip("the chunked scan needs rank_out == rank_in")
    print(f"[decode-prefill] case={case} L={L} L1={L1}", flush=True)
    t = workloads.to_device(prob)
    d1 = dict(prob["desc"], seqlen=L1)
    t1 = {k: (v[:, :L1].contiguous() if k in ("x", "B", "C", "dt", "beta", "gamma") else v)
          for k, v in t.items()}
    y1, _, state = ssm.forward(d1, prob["dtype"], t1["x"], t1["B"], t1["C"], t1["dt"], t1["A"],
                               omega=t1.get("omega"), beta=t1.get("beta"),
                               gamma=t1.get("gamma"), D=t1.get("D"), return_final_state=True)
    y2 = _steps(prob, t, state, L1, L)
    torch.cuda.synchronize()
    yr, hr = oracle.fwd(prob)
    e1 = rel_l2(_np(y1), yr[:, :L1])
    e2 = rel_l2(y2, yr[:, L1:])
    eh = rel_l2(_np(state), hr)
    print(f"[decode-prefill] case={case} prefill={e1:.2e} steps={e2:.2e} state={eh:.2e}",
          flush=True)
    assert e1 <= tol(prob) and e2 <= tol(prob) and eh <= tol(prob), (e1, e2, eh)


def test_decode_is_reproducible_and_leaves_inputs():
    name, kw = CASES["bf16_hybrid"]
    prob = workloads.make_problem(workloads.spec(name, seqlen=2, **kw), seed=19)
    h0 = workloads.make_state(prob["desc"], seed=23)
    t = workloads.to_device(prob)
    outs = []
    for _ in range(2):
        state = torch.from_numpy(h0).cuda()
        y = _steps(prob, t, state, 0, 2)
        outs.append((y, _np(state)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("tps", [64, 128, 256])
@pytest.mark.parametrize("case", ["f32_hybrid", "bf16_ssd_mimo", "f32_siso"])
def test_decode_slices_per_workgroup(case, tps, monkeypatch):
    """1, 2 or 4 slices share a workgroup (the library picks by state size; the
    override forces each), including a tail workgroup with fewer live slices."""
    name, kw = CASES[case]
    kw = dict(kw, batch=3)
    prob = workloads.make_problem(workloads.spec(name, seqlen=3, **kw), seed=29)
    if prob["desc"]["headdim"] // 4 > tps:
        pytest.skip("a state row needs more threads than the slice has")
    monkeypatch.setenv("SSM_DECODE_TPS", str(tps))
    h0 = workloads.make_state(prob["desc"], seed=31, scale=0.5)
    print(f"[decode-tps] case={case} tps={tps}", flush=True)
    t = workloads.to_device(prob)
    state = torch.from_numpy(h0).cuda()
    y = _steps(prob, t, state, 0, 3)
    yr, hr = oracle.fwd(prob, h0=h0.astype(np.float64))
    ey, eh = rel_l2(y, yr), rel_l2(_np(state), hr)
    print(f"[decode-tps] case={case} tps={tps} y={ey:.2e} state={eh:.2e}", flush=True)
    assert ey <= tol(prob) and eh <= tol(prob), (ey, eh)
