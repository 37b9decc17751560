"""GPU parity of the reverse-mode pass against the fp64 oracle's adjoint.

Every gradient tensor (dx, dB, dC, ddt, dA, domega, dbeta, dgamma, dD) is
compared by relative L2: 1e-4 on the fp32 path, 1e-2 on the bf16 path.
Full-size workloads are checked on sampled (batch, head) slices for the
per-token gradients.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import rel_l2, run_bwd, tol

pytestmark = pytest.mark.gpu

GRADS = ["dx", "dB", "dC", "ddt", "dA", "domega", "dbeta", "dgamma", "dD"]

SMALL = {
    "f32_siso_full": ("siso_f32", dict()),
    "f32_siso_ragged": ("siso_f32", dict(batch=2, seqlen=200, nheads=3, ngroups=3)),
    "f32_head_n32": ("ssd_siso", dict(dtype="f32", dstate=32, n_real=32, headdim=16, batch=2,
                                      nheads=2, ngroups=2, seqlen=150)),
    "f32_head_r2": ("ssd_mimo", dict(dtype="f32", dstate=32, n_real=32, headdim=16, rank_in=2,
                                     rank_out=2, batch=2, nheads=2, ngroups=2, seqlen=100)),
    "f32_hybrid_r2": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_pairs=8, headdim=16,
                                     batch=2, nheads=2, ngroups=2, seqlen=77)),
    "f32_hybrid_r1": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_pairs=8, headdim=16,
                                     rank_in=1, rank_out=1, batch=2, nheads=2, ngroups=2,
                                     seqlen=70)),
    "f32_hybrid_n16": ("hybrid", dict(dtype="f32", dstate=16, n_real=8, n_pairs=4, headdim=16,
                                      rank_in=1, rank_out=1, batch=1, nheads=2, ngroups=2,
                                      seqlen=90)),
    "f32_coord_plain_r1": ("hybrid", dict(dtype="f32", two_endpoint=False, dstate=32,
                                          n_real=16, n_pairs=8, headdim=16, rank_in=1,
                                          rank_out=1, batch=2, nheads=2, ngroups=2, seqlen=75)),
    "f32_coord_plain_r2": ("hybrid", dict(dtype="f32", two_endpoint=False, dstate=32,
                                          n_real=16, n_pairs=8, headdim=16, batch=2, nheads=2,
                                          ngroups=2, seqlen=61)),
    "bf16_ssd_siso": ("ssd_siso", dict(batch=2, seqlen=300, nheads=2, ngroups=2)),
    "bf16_ssd_siso_n64": ("ssd_siso", dict(batch=2, seqlen=130, nheads=2, ngroups=2, dstate=64,
                                           n_real=64)),
    "bf16_ssd_mimo": ("ssd_mimo", dict(batch=2, seqlen=200, nheads=2, ngroups=2)),
    "bf16_hybrid": ("hybrid", dict(batch=2, seqlen=150, nheads=2, ngroups=2)),
    "bf16_hybrid_r1": ("hybrid_r1", dict(batch=2, seqlen=150, nheads=2, ngroups=2)),
    "bf16_len_chunk1": ("hybrid", dict(batch=1, seqlen=17, nheads=2, ngroups=2)),
    # B / C groups shared by several heads: dB / dC sum over the group's heads
    "f32_groups_siso": ("ssd_siso", dict(dtype="f32", dstate=32, n_real=32, headdim=16, batch=2,
                                         nheads=4, ngroups=2, seqlen=150)),
    "f32_groups_hybrid": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_pairs=8,
                                         headdim=16, batch=2, nheads=3, ngroups=1, seqlen=77)),
    "bf16_groups_siso": ("ssd_siso", dict(batch=2, seqlen=130, nheads=4, ngroups=2)),
    "bf16_groups_mimo": ("ssd_mimo", dict(batch=1, seqlen=200, nheads=4, ngroups=1)),
    "bf16_groups_hybrid": ("hybrid", dict(batch=2, seqlen=150, nheads=4, ngroups=2)),
    "bf16_groups_hybrid_r1": ("hybrid_r1", dict(batch=1, seqlen=90, nheads=6, ngroups=3)),
    # HybridMamba row mixes: real rows only, rotating pairs only, a quarter of the rows paired
    "bf16_hm_real_only": ("hybrid", dict(batch=2, seqlen=150, nheads=2, ngroups=2, n_real=64,
                                         n_pairs=0)),
    "bf16_hm_pairs_only": ("hybrid", dict(batch=2, seqlen=150, nheads=2, ngroups=2, n_real=0,
                                          n_pairs=32)),
    "bf16_hm_quarter_pairs": ("hybrid", dict(batch=2, seqlen=150, nheads=2, ngroups=2,
                                             n_real=48, n_pairs=8)),
    "f32_hm_pairs_only": ("hybrid", dict(dtype="f32", dstate=32, n_real=0, n_pairs=16,
                                         headdim=16, batch=2, nheads=2, ngroups=2, seqlen=77)),
    # write and readout widths that differ (O != R; no feedthrough then)
    "f32_head_r2o1": ("ssd_mimo", dict(dtype="f32", dstate=32, n_real=32, headdim=16, rank_in=2,
                                       rank_out=1, has_D=False, batch=2, nheads=2, ngroups=2,
                                       seqlen=100)),
    "f32_hybrid_r1o2": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_pairs=8, headdim=16,
                                       rank_in=1, rank_out=2, has_D=False, batch=2, nheads=2,
                                       ngroups=2, seqlen=77)),
    "bf16_mimo_r4o2": ("ssd_mimo", dict(batch=2, seqlen=130, nheads=2, ngroups=2, rank_in=4,
                                        rank_out=2, has_D=False)),
    "bf16_mimo_r1o4": ("ssd_mimo", dict(batch=2, seqlen=130, nheads=2, ngroups=2, rank_in=1,
                                        rank_out=4, has_D=False)),
    "bf16_hybrid_r2o1": ("hybrid", dict(batch=2, seqlen=150, nheads=4, ngroups=2, rank_in=2,
                                        rank_out=1, has_D=False)),
}


def compare(prob, g, ref, slices=None):
    errs = {}
    for k in GRADS:
        if k not in g or ref.get(k) is None:
            continue
        a, r = g[k], ref[k]
        if slices is not None:
            if k in ("dA", "domega", "dD"):
                continue
            a = np.stack([a[b, :, h] for b, h in slices])
            r = np.stack([r[b, :, h] for b, h in slices])
        errs[k] = rel_l2(a, r)
    return errs


@pytest.mark.parametrize("case", sorted(SMALL))
def test_bwd_small_matches_oracle(case):
    name, kw = SMALL[case]
    prob = workloads.make_problem(workloads.spec(name, **kw), seed=0, with_dy=True)
    print(f"[bwd] case={case} desc={prob['desc']}", flush=True)
    _, g = run_bwd(prob)
    ref = oracle.bwd(prob, prob["dy"])
    errs = compare(prob, g, ref)
    print(f"[bwd] case={case} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol(prob)}
    assert not bad, bad


@pytest.mark.parametrize("name", ["hybrid_bwd", "ssd_mimo_bwd", "ssd_siso"])
def test_bwd_full_size_sampled_slices(name):
    prob = workloads.make_problem(name, seed=0, with_dy=True)
    d = prob["desc"]
    print(f"[bwd-full] {name} desc={d}", flush=True)
    _, g = run_bwd(prob)
    rng = np.random.default_rng(2)
    slices = sorted({(int(rng.integers(d["batch"])), int(rng.integers(d["nheads"])))
                     for _ in range(4)} | {(0, 0), (d["batch"] - 1, d["nheads"] - 1)})
    ref = oracle.bwd(prob, prob["dy"], slices=slices)
    errs = compare(prob, g, ref, slices=slices)
    print(f"[bwd-full] {name} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol(prob)}
    assert not bad, bad
    for k, v in g.items():
        assert np.isfinite(v).all(), k


def test_bwd_deterministic():
    prob = workloads.make_problem(workloads.spec("hybrid", batch=2, seqlen=300, nheads=2,
                                                 ngroups=2), seed=4, with_dy=True)
    _, g1 = run_bwd(prob)
    _, g2 = run_bwd(prob)
    for k in g1:
        assert np.array_equal(g1[k], g2[k]), k
