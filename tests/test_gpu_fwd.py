"""GPU parity of the forward scan against the fp64 oracle (relative L2 per tensor).

Tolerances: 1e-4 for the fp32 path, 1e-2 for the bf16 path.  Small shapes use
ragged lengths (not a multiple of the chunk) and several chunks; full-size
workloads are checked on sampled (batch, head) slices, which the oracle
computes independently of the rest.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import rel_l2, rel_l2_by_position, run_fwd, tol

pytestmark = pytest.mark.gpu


SMALL_CASES = {
    # fp32 path: the same kernels as bf16 with fp32 operands, checked at 1e-4
    "f32_siso_full": ("siso_f32", {}),
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
                                          rank_out=1, batch=2, nheads=2, ngroups=2,
                                          seqlen=75)),
    "f32_coord_plain_r2": ("hybrid", dict(dtype="f32", two_endpoint=False, dstate=32,
                                          n_real=16, n_pairs=8, headdim=16, batch=2, nheads=2,
                                          ngroups=2, seqlen=61)),
    # bf16 path
    "bf16_ssd_siso": ("ssd_siso", dict(batch=2, seqlen=300, nheads=3, ngroups=3)),
    "bf16_ssd_siso_n64": ("ssd_siso", dict(batch=2, seqlen=130, nheads=2, ngroups=2, dstate=64,
                                           n_real=64)),
    "bf16_ssd_mimo": ("ssd_mimo", dict(batch=2, seqlen=200, nheads=2, ngroups=2)),
    "bf16_hybrid": ("hybrid", dict(batch=2, seqlen=150, nheads=2, ngroups=2)),
    "bf16_hybrid_r1": ("hybrid_r1", dict(batch=2, seqlen=150, nheads=2, ngroups=2)),
    "bf16_groups": ("ssd_siso", dict(batch=1, seqlen=100, nheads=4, ngroups=2, dstate=64,
                                     n_real=64)),
    "bf16_len1": ("ssd_siso", dict(batch=2, seqlen=1, nheads=2, ngroups=2, dstate=64,
                                   n_real=64)),
    "bf16_len_chunk": ("ssd_siso", dict(batch=1, seqlen=64, nheads=2, ngroups=2, dstate=64,
                                        n_real=64)),
    "bf16_len_chunk1": ("hybrid", dict(batch=1, seqlen=17, nheads=2, ngroups=2)),
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
    # the pairs of a head decaying at different rates (one rate per (head, pair))
    "f32_hybrid_pair_rates": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_pairs=8,
                                             headdim=16, batch=2, nheads=2, ngroups=2,
                                             seqlen=77, pair_rate_per_pair=True)),
    "f32_pairs_only_pair_rates": ("hybrid", dict(dtype="f32", dstate=32, n_real=0, n_pairs=16,
                                                 headdim=16, rank_in=1, rank_out=1, batch=1,
                                                 nheads=2, ngroups=2, seqlen=70,
                                                 pair_rate_per_pair=True)),
    "bf16_hybrid_pair_rates": ("hybrid", dict(batch=2, seqlen=150, nheads=2, ngroups=2,
                                              pair_rate_per_pair=True)),
    "bf16_hybrid_r1_pair_rates": ("hybrid_r1", dict(batch=2, seqlen=150, nheads=2, ngroups=2,
                                                    pair_rate_per_pair=True)),
    # steps given directly (no softplus in the kernel), positive
    "f32_head_no_softplus": ("ssd_siso", dict(dtype="f32", dstate=32, n_real=32, headdim=16,
                                              batch=2, nheads=2, ngroups=2, seqlen=150,
                                              dt_softplus=False, dt_mean=0.1, dt_std=0.02)),
    "f32_hybrid_no_softplus": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_pairs=8,
                                              headdim=16, batch=2, nheads=2, ngroups=2,
                                              seqlen=77, dt_softplus=False, dt_mean=0.1,
                                              dt_std=0.02)),
    "bf16_ssd_siso_no_softplus": ("ssd_siso", dict(batch=2, seqlen=300, nheads=2, ngroups=2,
                                                   dt_softplus=False, dt_mean=0.1,
                                                   dt_std=0.02)),
    "bf16_mimo_no_softplus": ("ssd_mimo", dict(batch=2, seqlen=200, nheads=2, ngroups=2,
                                               dt_softplus=False, dt_mean=0.1, dt_std=0.02)),
    "bf16_hybrid_no_softplus": ("hybrid", dict(batch=2, seqlen=150, nheads=2, ngroups=2,
                                               dt_softplus=False, dt_mean=0.1, dt_std=0.02)),
    # steep per-row decay: steps ~ softplus(N(2, 0.5)) with rates 16 (a row decays by
    # ~e^-34 per token), so every chunk is redone token by token; and spike mixes, where
    # some ranges and chunks stay on the chunked path and others are redone
    "f32_hybrid_steep": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_pairs=8,
                                        headdim=16, batch=2, nheads=2, ngroups=2, seqlen=77,
                                        dt_mean=2.0, A_lo=16.0, A_hi=16.0)),
    "f32_coord_plain_steep": ("hybrid", dict(dtype="f32", two_endpoint=False, dstate=32,
                                             n_real=16, n_pairs=8, headdim=16, batch=2,
                                             nheads=2, ngroups=2, seqlen=61, dt_mean=2.0,
                                             A_lo=16.0, A_hi=16.0)),
    "f32_hybrid_r1_steep": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_pairs=8,
                                           headdim=16, rank_in=1, rank_out=1, batch=2,
                                           nheads=2, ngroups=2, seqlen=70, dt_mean=2.0,
                                           A_lo=16.0, A_hi=16.0)),
    "bf16_hybrid_steep": ("hybrid", dict(batch=2, seqlen=150, nheads=2, ngroups=2, dt_mean=2.0,
                                         A_lo=16.0, A_hi=16.0)),
    "bf16_hybrid_r1_steep": ("hybrid_r1", dict(batch=2, seqlen=150, nheads=2, ngroups=2,
                                               dt_mean=2.0, A_lo=16.0, A_hi=16.0)),
    "bf16_hybrid_spikes": ("hybrid", dict(batch=2, seqlen=300, nheads=4, ngroups=4,
                                          dt_spike_prob=[0.0, 0.05, 0.3, 0.7], dt_spike_mean=3.0,
                                          pair_rate_per_pair=True)),
    "f32_hybrid_spikes": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_pairs=8,
                                         headdim=16, batch=2, nheads=4, ngroups=2, seqlen=150,
                                         dt_spike_prob=[0.0, 0.05, 0.3, 0.7],
                                         dt_spike_mean=3.0)),
    "bf16_te_head_steep": ("ssd_siso", dict(batch=2, seqlen=150, nheads=2, ngroups=2, dstate=64,
                                            n_real=64, two_endpoint=True, dt_mean=2.0,
                                            A_lo=16.0, A_hi=16.0, chunk=0)),
    # real static rows (decay e^{-A} per token whatever the step) next to dynamic rows and
    # pairs; HM-75 (three quarters of the rows in rotating pairs); static rows only; static
    # rates large enough that every chunk is redone token by token; static rates up to 6,
    # which put some chunks past the fold limit and leave others on the chunked path
    "f32_hybrid_static": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_static=8,
                                         n_pairs=8, headdim=16, batch=2, nheads=2, ngroups=2,
                                         seqlen=77)),
    "f32_coord_plain_static": ("hybrid", dict(dtype="f32", two_endpoint=False, dstate=32,
                                              n_real=16, n_static=16, n_pairs=8, headdim=16,
                                              batch=2, nheads=2, ngroups=2, seqlen=61)),
    "f32_hybrid_static_steep": ("hybrid", dict(dtype="f32", dstate=32, n_real=16, n_static=8,
                                               n_pairs=8, headdim=16, batch=2, nheads=2,
                                               ngroups=2, seqlen=77, A_static_lo=16.0,
                                               A_static_hi=16.0)),
    "bf16_hm75_static": ("hybrid", dict(batch=2, seqlen=150, nheads=2, ngroups=2, n_real=16,
                                        n_static=8, n_pairs=24)),
    "bf16_static_only": ("hybrid", dict(batch=2, seqlen=150, nheads=2, ngroups=2, n_real=64,
                                        n_static=64, n_pairs=0)),
    "bf16_hybrid_r1_static": ("hybrid_r1", dict(batch=2, seqlen=150, nheads=2, ngroups=2,
                                                n_static=16, A_static_hi=6.0)),
    # head decay needs no fallback (its masks and factors are exponents <= 0): a check
    "bf16_ssd_siso_steep": ("ssd_siso", dict(batch=2, seqlen=300, nheads=2, ngroups=2,
                                             dt_mean=2.0, A_lo=16.0, A_hi=16.0)),
    "bf16_mimo_steep": ("ssd_mimo", dict(batch=2, seqlen=200, nheads=2, ngroups=2, dt_mean=2.0,
                                         A_lo=16.0, A_hi=16.0)),
}


@pytest.mark.parametrize("case", sorted(SMALL_CASES))
def test_fwd_small_matches_oracle(case):
    name, kw = SMALL_CASES[case]
    prob = workloads.make_problem(workloads.spec(name, **kw), seed=0)
    print(f"[fwd] case={case} desc={prob['desc']}", flush=True)
    y, _, _ = run_fwd(prob)
    ref, _ = oracle.fwd(prob)
    err = rel_l2(y, ref)
    print(f"[fwd] case={case} rel_l2={err:.3e}", flush=True)
    assert err <= tol(prob), err


FULL = ["ssd_siso", "ssd_mimo", "hybrid", "hybrid_r1"]


@pytest.mark.parametrize("name", FULL)
@pytest.mark.parametrize("save", [False, True])
def test_fwd_full_size_whole_tensor(name, save):
    """The workload at its full size, in the launch configuration the bench times
    (save=False: the forward alone; save=True: the forward of a training step, which
    also writes the chunk-boundary states), against the oracle over every slice: one
    rel-L2 over the whole output, and one per token position inside a chunk."""
    prob = workloads.make_problem(name, seed=0)
    d = prob["desc"]
    print(f"[fwd-full] {name} save={save} desc={d}", flush=True)
    y, _, _ = run_fwd(prob, save=save)
    assert np.isfinite(y).all()
    ref, _ = oracle.fwd(prob)
    err = rel_l2(y, ref)
    pos = rel_l2_by_position(y, ref, 64)
    print(f"[fwd-full] {name} save={save} rel_l2={err:.3e} worst position "
          f"{int(pos.argmax())}: {pos.max():.3e}", flush=True)
    assert err <= tol(prob), err
    assert pos.max() <= tol(prob), pos


def test_fwd_deterministic():
    prob = workloads.make_problem(workloads.spec("hybrid", batch=2, seqlen=500, nheads=4,
                                                 ngroups=4), seed=3)
    y1, _, _ = run_fwd(prob)
    y2, _, _ = run_fwd(prob)
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("name,kw,chunks", [
    ("ssd_siso", dict(batch=2, seqlen=300, nheads=2, ngroups=2, dstate=64, n_real=64), (32, 64)),
    ("ssd_mimo", dict(batch=2, seqlen=200, nheads=2, ngroups=2), (8, 16)),
    ("hybrid", dict(batch=2, seqlen=150, nheads=2, ngroups=2), (8, 16)),
])
def test_fwd_chunk_size_invariance(name, kw, chunks):
    prob = workloads.make_problem(workloads.spec(name, **kw), seed=5)
    ref, _ = oracle.fwd(prob)
    ys = []
    for q in chunks:
        y, _, _ = run_fwd(prob, chunk=q)
        err = rel_l2(y, ref)
        print(f"[chunk] {name} chunk={q} rel_l2={err:.3e}", flush=True)
        assert err <= tol(prob)
        ys.append(y)
    assert rel_l2(ys[0], ys[1]) <= tol(prob)


def test_fwd_siso_recovery_cross_kernel():
    # head decay routed through the per-row kernel (two-endpoint flag with
    # beta = 0, gamma = 1) reproduces the head-decay SSD kernel: the exact SISO
    # special case of the HybridMamba construction.
    prob = workloads.make_problem(workloads.spec("ssd_siso", batch=2, seqlen=130, nheads=2,
                                                 ngroups=2, dstate=64, n_real=64), seed=7)
    y_head, _, _ = run_fwd(prob)
    te = dict(prob)
    te["desc"] = dict(prob["desc"], two_endpoint=True)
    te["beta"] = np.zeros_like(prob["dt"])
    te["gamma"] = np.ones_like(prob["dt"])
    te["chunk"] = 0  # the per-row kernel's own chunk
    y_coord, _, _ = run_fwd(te)
    ref, _ = oracle.fwd(prob)
    assert rel_l2(y_head, ref) <= 1e-2 and rel_l2(y_coord, ref) <= 1e-2
    assert rel_l2(y_coord, y_head) <= 1e-2


def test_fwd_empty_is_noop():
    prob = workloads.make_problem(workloads.spec("ssd_siso", batch=1, seqlen=0, nheads=2,
                                                 ngroups=2, dstate=64, n_real=64), seed=0)
    y, _, _ = run_fwd(prob)
    assert y.size == 0
