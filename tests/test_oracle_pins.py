"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each test names the part of the recurrence it pins and what fixes it.  None of
them re-types the oracle's own loop: they compare against closed forms, library
routines (cumsum, lfilter, matmul, SVD), the O(L^2) form of Theorem 24 built
from explicit transfer products, the complex-diagonal form of Theorem 8, and
torch autograd of that O(L^2) form.

Page references: "When a Diagonal State Is Not Enough" (sungsoo.github.io),
Part 01 (recurrence, local retrieval rank), Part 03 (Theorem 8, Theorem 24,
SISO vs MIMO), Part 04 (exact recovery of SISO special cases), Part 08.2
(transfer C_t Phi_{t,s} B_s); arXiv abstract on mlinfo.pages.dev (HybridMamba,
SSD-MIMO).
"""
import math

import numpy as np
import pytest
import scipy.signal
import torch

import oracle
import workloads
from oracle import forms


def small(name, **kw):
    kw.setdefault("dtype", "f32")
    return workloads.spec(name, **kw)


def T64(a):
    return torch.tensor(np.asarray(a), dtype=torch.float64)


def scalar_problem(T, a, B, X, C=None, beta=None, gamma=None):
    """N = P = R = O = 1, head decay with constant a = exp(-dt * A), dt given directly."""
    desc = dict(batch=1, seqlen=T, nheads=1, ngroups=1, headdim=1, dstate=1, rank_in=1,
                rank_out=1, n_real=1, n_pairs=0, decay_mode="head", dt_softplus=False,
                two_endpoint=beta is not None, has_D=False)
    lam = -math.log(a) if a > 0 else 0.0
    dt = np.full((1, T, 1), 1.0, np.float32)
    A = np.array([lam], np.float32)
    C = np.ones(T, np.float32) if C is None else np.asarray(C, np.float32)
    p = dict(desc=desc, x=np.asarray(X, np.float32).reshape(1, T, 1, 1, 1),
             B=np.asarray(B, np.float32).reshape(1, T, 1, 1, 1),
             C=C.reshape(1, T, 1, 1, 1), dt=dt, A=A, omega=np.zeros((1, 0), np.float32),
             beta=None if beta is None else np.asarray(beta, np.float32).reshape(1, T, 1),
             gamma=None if gamma is None else np.asarray(gamma, np.float32).reshape(1, T, 1),
             D=None)
    return p, float(np.exp(-np.float64(np.float32(lam))))


# ---------------------------------------------------------------- P1 closed forms
def test_p1_impulse_response_is_geometric(oracle_lib):
    T, s = 20, 3
    X = np.zeros(T); X[s] = 1.0
    p, a = scalar_problem(T, 0.8, np.ones(T), X)
    y, _ = oracle.fwd(p)
    y = y.reshape(T)
    expect = np.array([a ** (t - s) if t >= s else 0.0 for t in range(T)])
    np.testing.assert_allclose(y, expect, rtol=1e-12, atol=1e-15)


def test_p1_unit_decay_is_cumsum(oracle_lib):
    rng = np.random.default_rng(3)
    T = 33
    Bv = rng.standard_normal(T).astype(np.float32)
    X = rng.standard_normal(T).astype(np.float32)
    p, _ = scalar_problem(T, 1.0, Bv, X)
    y, _ = oracle.fwd(p)
    np.testing.assert_allclose(y.reshape(T), np.cumsum(Bv.astype(np.float64) * X), rtol=1e-12)


def test_p1_unit_decay_is_causal_linear_attention(oracle_lib):
    # a == 1 with general B_t, C_t: y = tril(C B^T) X, an unnormalized causal
    # linear attention (Theorem 24 with an all-ones mask).
    rng = np.random.default_rng(4)
    T, N, P = 17, 5, 3
    desc = dict(batch=1, seqlen=T, nheads=1, ngroups=1, headdim=P, dstate=N, rank_in=1,
                rank_out=1, n_real=N, n_pairs=0, decay_mode="head", dt_softplus=False,
                two_endpoint=False, has_D=False)
    Bm = rng.standard_normal((T, N)).astype(np.float32)
    Cm = rng.standard_normal((T, N)).astype(np.float32)
    X = rng.standard_normal((T, P)).astype(np.float32)
    p = dict(desc=desc, x=X.reshape(1, T, 1, 1, P), B=Bm.reshape(1, T, 1, 1, N),
             C=Cm.reshape(1, T, 1, 1, N), dt=np.ones((1, T, 1), np.float32),
             A=np.zeros(1, np.float32), omega=np.zeros((1, 0), np.float32),
             beta=None, gamma=None, D=None)
    y, _ = oracle.fwd(p)
    att = np.tril(Cm.astype(np.float64) @ Bm.astype(np.float64).T)
    np.testing.assert_allclose(y.reshape(T, P), att @ X.astype(np.float64), rtol=1e-11,
                               atol=1e-12)


def test_p1_constant_decay_is_first_order_iir(oracle_lib):
    rng = np.random.default_rng(5)
    T = 64
    Bv = rng.standard_normal(T).astype(np.float32)
    X = rng.standard_normal(T).astype(np.float32)
    p, a = scalar_problem(T, 0.9, Bv, X)
    y, _ = oracle.fwd(p)
    ref = scipy.signal.lfilter([1.0], [1.0, -a], Bv.astype(np.float64) * X)
    np.testing.assert_allclose(y.reshape(T), ref, rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------- P2 Theorem 24 form
@pytest.mark.parametrize("name,kw", [
    ("ssd_siso", dict(batch=2, seqlen=8, nheads=3, ngroups=3, headdim=3, dstate=4, n_real=4)),
    ("ssd_mimo", dict(batch=1, seqlen=7, nheads=2, ngroups=1, headdim=2, dstate=4, n_real=4,
                      rank_in=3, rank_out=3)),
    ("hybrid", dict(batch=2, seqlen=8, nheads=2, ngroups=2, headdim=3, dstate=6, n_real=2,
                    n_pairs=2, rank_in=2, rank_out=2)),
    # the pairs of a head decaying at different rates ("different decay laws", arXiv abstract)
    ("hybrid", dict(batch=1, seqlen=8, nheads=2, ngroups=2, headdim=2, dstate=8, n_real=2,
                    n_pairs=3, rank_in=2, rank_out=2, pair_rate_per_pair=True)),
    # real static, real dynamic and complex dynamic rows in one head (Part 08 section 3)
    ("hybrid", dict(batch=2, seqlen=8, nheads=2, ngroups=2, headdim=2, dstate=10, n_real=4,
                    n_static=2, n_pairs=3, rank_in=2, rank_out=2, pair_rate_per_pair=True)),
])
def test_p2_recurrence_equals_quadratic_form(oracle_lib, name, kw):
    p = workloads.make_problem(small(name, **kw), seed=11)
    d = p["desc"]
    rng = np.random.default_rng(12)
    h0 = rng.standard_normal((d["batch"], d["nheads"], d["dstate"], d["headdim"]))
    y, _ = oracle.fwd(p, h0=h0)
    om = p["omega"] if d["n_pairs"] else np.zeros((d["nheads"], 1), np.float32)
    yq = forms.quadratic_y(d, T64(p["x"]), T64(p["B"]), T64(p["C"]), T64(p["dt"]), T64(p["A"]),
                           T64(om), None if p["beta"] is None else T64(p["beta"]),
                           None if p["gamma"] is None else T64(p["gamma"]),
                           None if p["D"] is None else T64(p["D"]), h0=T64(h0)).numpy()
    np.testing.assert_allclose(y, yq, rtol=1e-10, atol=1e-12 * np.abs(yq).max())


def test_p2_output_rank_mismatch_supported(oracle_lib):
    # O != R (SSD-MIMO supports different input / output widths; Part 08.3)
    s = small("ssd_mimo", batch=1, seqlen=6, nheads=1, ngroups=1, headdim=2, dstate=4,
              n_real=4, rank_in=3, rank_out=2, has_D=False)
    p = workloads.make_problem(s, seed=2)
    y, _ = oracle.fwd(p)
    d = p["desc"]
    yq = forms.quadratic_y(d, T64(p["x"]), T64(p["B"]), T64(p["C"]), T64(p["dt"]),
                           T64(p["A"])).numpy()
    np.testing.assert_allclose(y, yq, rtol=1e-10, atol=1e-14)


# ---------------------------------------------------------------- P3 complex pairs
@pytest.mark.parametrize("per_pair", [False, True])
def test_p3_real_pairs_equal_complex_diagonal(oracle_lib, per_pair):
    p = workloads.make_problem(small("hybrid", batch=2, seqlen=12, nheads=2, ngroups=2,
                                     headdim=3, dstate=10, n_real=4, n_pairs=3,
                                     pair_rate_per_pair=per_pair), seed=21)
    if per_pair:
        assert len(np.unique(p["A"][0, 4:])) == 3  # three distinct pair rates in one head
    y, _ = oracle.fwd(p)
    yc = forms.complex_y(p["desc"], p["x"], p["B"], p["C"], p["dt"], p["A"], p["omega"],
                         p["beta"], p["gamma"], p["D"])
    np.testing.assert_allclose(y, yc, rtol=1e-10, atol=1e-13)


def test_p3_single_pair_impulse_closed_form(oracle_lib):
    T, s = 25, 4
    desc = dict(batch=1, seqlen=T, nheads=1, ngroups=1, headdim=1, dstate=2, rank_in=1,
                rank_out=1, n_real=0, n_pairs=1, decay_mode="coord", dt_softplus=False,
                two_endpoint=False, has_D=False)
    dt, rate, om = 0.5, 0.3, 1.1
    X = np.zeros((1, T, 1, 1, 1), np.float32); X[0, s] = 1.0
    Bm = np.zeros((1, T, 1, 1, 2), np.float32); Bm[..., 0] = 1.0   # write e_0
    for ci, fn in ((0, np.cos), (1, np.sin)):
        Cm = np.zeros((1, T, 1, 1, 2), np.float32); Cm[..., ci] = 1.0
        p = dict(desc=desc, x=X, B=Bm, C=Cm, dt=np.full((1, T, 1), dt, np.float32),
                 A=np.array([[rate]], np.float32), omega=np.array([[om]], np.float32),
                 beta=None, gamma=None, D=None)
        y, _ = oracle.fwd(p)
        d64 = np.float64(np.float32(dt))
        rho = np.exp(-d64 * np.float64(np.float32(rate)))
        th = d64 * np.float64(np.float32(om))
        k = np.arange(T) - s
        expect = np.where(k >= 0, rho ** np.maximum(k, 0) * fn(np.maximum(k, 0) * th), 0.0)
        np.testing.assert_allclose(y.reshape(T), expect, rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- P4 fixed-basis invariance
def test_p4_fixed_basis_change_leaves_outputs_unchanged(oracle_lib):
    # A fixed S commuting with every A_t (positive scaling on real rows, a scaled
    # rotation on each pair) maps B -> S B and C -> S^{-T} C with y unchanged
    # (fixed-basis diagonal equivalence, Part 01).
    p = workloads.make_problem(small("hybrid", batch=1, seqlen=10, nheads=2, ngroups=2,
                                     headdim=2, dstate=6, n_real=2, n_pairs=2), seed=31)
    d = p["desc"]
    N, nr = d["dstate"], d["n_real"]
    rng = np.random.default_rng(32)
    S = np.zeros((N, N))
    for n in range(nr):
        S[n, n] = rng.uniform(0.5, 2.0)
    for k in range(d["n_pairs"]):
        i = nr + 2 * k
        sc, ph = rng.uniform(0.5, 2.0), rng.uniform(-math.pi, math.pi)
        S[i:i + 2, i:i + 2] = sc * np.array([[math.cos(ph), -math.sin(ph)],
                                             [math.sin(ph), math.cos(ph)]])
    q = dict(p)
    # B[..., r, :] is the column B_t e_r of the N x R map
    q["B"] = np.einsum("nm,btgrm->btgrn", S, p["B"].astype(np.float64)).astype(np.float32)
    q["C"] = np.einsum("nm,btgom->btgon", np.linalg.inv(S).T,
                       p["C"].astype(np.float64)).astype(np.float32)
    # the fp32 storage of the transformed maps is inexact; compare against the
    # fp64 transform via the quadratic form of the rounded inputs instead of y
    y_orig = forms.quadratic_y(d, T64(p["x"]), T64(np.einsum("nm,btgrm->btgrn", S, p["B"])),
                               T64(np.einsum("nm,btgom->btgon", np.linalg.inv(S).T, p["C"])),
                               T64(p["dt"]), T64(p["A"]), T64(p["omega"]), T64(p["beta"]),
                               T64(p["gamma"]), T64(p["D"])).numpy()
    y_base, _ = oracle.fwd(p)
    np.testing.assert_allclose(y_orig, y_base, rtol=1e-9, atol=1e-12)
    y_tr, _ = oracle.fwd(q)
    np.testing.assert_allclose(y_tr, y_base, rtol=1e-5, atol=1e-6 * np.abs(y_base).max())


# ---------------------------------------------------------------- P5 two-endpoint write
def test_p5_plain_write_is_two_endpoint_with_beta0_gamma1(oracle_lib):
    s = small("hybrid", batch=2, seqlen=9, nheads=2, ngroups=2, headdim=3, dstate=6,
              n_real=2, n_pairs=2)
    p = workloads.make_problem(s, seed=41)
    q = dict(p)
    q["desc"] = dict(p["desc"], two_endpoint=False)
    q["beta"] = q["gamma"] = None
    r = dict(p)
    r["beta"] = np.zeros_like(p["beta"])
    r["gamma"] = np.ones_like(p["gamma"])
    y_plain, h_plain = oracle.fwd(q)
    y_te, h_te = oracle.fwd(r)
    assert np.array_equal(y_plain, y_te) and np.array_equal(h_plain, h_te)


def test_p5_scalar_two_endpoint_closed_form(oracle_lib):
    T, s = 12, 2
    rng = np.random.default_rng(51)
    beta = rng.uniform(0.1, 0.9, T)
    gamma = rng.uniform(0.1, 0.9, T)
    X = np.zeros(T); X[s] = 1.0
    p, a = scalar_problem(T, 0.7, np.ones(T), X, beta=beta, gamma=gamma)
    y, _ = oracle.fwd(p)
    bt, gm = p["beta"].reshape(T).astype(np.float64), p["gamma"].reshape(T).astype(np.float64)
    expect = np.zeros(T)
    expect[s] = gm[s]
    for t in range(s + 1, T):
        expect[t] = a ** (t - s - 1) * (gm[s] * a + bt[s + 1])
    np.testing.assert_allclose(y.reshape(T), expect, rtol=1e-12, atol=1e-15)


def test_p5_golden_scalar_two_endpoint(oracle_lib):
    # hand-derived values, tests/golden/scalar_two_endpoint_impulse.txt
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "scalar_two_endpoint_impulse.txt")
    vals = [float(v) for v in open(path).read().split("---")[1].split()]
    T = len(vals)
    X = np.zeros(T); X[1] = 1.0
    beta = np.full(T, 0.25); gamma = np.full(T, 0.5)
    p, _ = scalar_problem(T, 0.5, np.ones(T), X, beta=beta, gamma=gamma)
    y, _ = oracle.fwd(p)
    np.testing.assert_allclose(y.reshape(T), vals, rtol=1e-6, atol=1e-12)


def test_p5_shift_identity(oracle_lib):
    # h'_t = h_t - gamma_t B_t X_t obeys h'_t = A_t h'_{t-1} + (gamma_{t-1} A_t + beta_t) B_{t-1} X_{t-1}
    # and y_t = C_t^T h'_t + gamma_t C_t^T B_t X_t + D X_t: a plain recurrence with
    # shifted writes.  Built here with explicit matrices from the O(L^2) helper.
    s = small("hybrid", batch=1, seqlen=9, nheads=1, ngroups=1, headdim=2, dstate=4,
              n_real=2, n_pairs=1, rank_in=1, rank_out=1)
    p = workloads.make_problem(s, seed=53)
    d = p["desc"]
    y, _ = oracle.fwd(p)
    Am = forms.transition_matrices(d, T64(p["dt"]), T64(p["A"]), T64(p["omega"])).numpy()
    x, Bm, Cm = (p[k].astype(np.float64) for k in ("x", "B", "C"))
    bt, gm = p["beta"].astype(np.float64), p["gamma"].astype(np.float64)
    hp = np.zeros((d["dstate"], d["headdim"]))
    for t in range(d["seqlen"]):
        hp = Am[0, t, 0] @ hp
        if t > 0:
            w = Bm[0, t - 1, 0].T @ x[0, t - 1, 0]
            hp = hp + (gm[0, t - 1, 0] * Am[0, t, 0] + bt[0, t, 0] * np.eye(d["dstate"])) @ w
        wt = Bm[0, t, 0].T @ x[0, t, 0]
        yt = Cm[0, t, 0] @ hp + gm[0, t, 0] * (Cm[0, t, 0] @ wt) + p["D"][0] * x[0, t, 0]
        np.testing.assert_allclose(y[0, t, 0], yt, rtol=1e-10, atol=1e-13)


# ---------------------------------------------------------------- P6 retrieval rank
@pytest.mark.parametrize("O,rankB", [(1, 4), (2, 4), (4, 1), (4, 2), (4, 4), (2, 1)])
def test_p6_local_retrieval_rank_bound(oracle_lib, O, rankB):
    # Theorem 21 (Part 01, Part 08.2): rank of the s -> t transfer is at most
    # min(O, rank B_s), and generic readouts attain it.
    R, N, T = 4, 8, 6
    rng = np.random.default_rng(61 + 10 * O + rankB)
    desc = dict(batch=1, seqlen=T, nheads=1, ngroups=1, headdim=1, dstate=N, rank_in=R,
                rank_out=O, n_real=N, n_pairs=0, decay_mode="coord", dt_softplus=False,
                two_endpoint=False, has_D=False)
    # decays in [0.5, 0.99]
    a = rng.uniform(0.5, 0.99, N)
    A = (-np.log(a)).astype(np.float32).reshape(1, N)
    Bm = rng.standard_normal((1, T, 1, R, N))
    s = 1
    # integer factors keep the product exactly rank-deficient after fp32 storage
    Bm[0, s, 0] = (rng.integers(-3, 4, (R, rankB)) @ rng.integers(-3, 4, (rankB, N)))
    assert np.linalg.matrix_rank(Bm[0, s, 0]) == rankB
    Cm = rng.standard_normal((1, T, 1, O, N))
    base = dict(desc=desc, B=Bm.astype(np.float32), C=Cm.astype(np.float32),
                dt=np.ones((1, T, 1), np.float32), A=A, omega=np.zeros((1, 0), np.float32),
                beta=None, gamma=None, D=None)
    for t in range(s, T):
        J = np.zeros((O, R))
        for r in range(R):
            X = np.zeros((1, T, 1, R, 1), np.float32)
            X[0, s, 0, r, 0] = 1.0
            y, _ = oracle.fwd(dict(base, x=X))
            J[:, r] = y[0, t, 0, :, 0]
        Jref = forms.transfer(desc, base["B"], base["C"], base["dt"], base["A"],
                              np.zeros((1, 1)), None, None, 0, 0, t, s)
        np.testing.assert_allclose(J, Jref, rtol=1e-10, atol=1e-12)
        sv = np.linalg.svd(J, compute_uv=False)
        rank = int((sv > 1e-9 * sv[0]).sum())
        assert rank == min(O, rankB)


# ---------------------------------------------------------------- P7 SISO recovery
def test_p7_siso_recovery_is_bitwise(oracle_lib):
    # The general (per-row rate) oracle with R = O = 1, no pairs, beta = 0, gamma = 1
    # and A_{h,n} = A_h reproduces the head-decay SISO oracle bit for bit
    # (exact special-case recovery, abstract and Part 04).
    s = small("ssd_siso", batch=2, seqlen=40, nheads=3, ngroups=3, headdim=4, dstate=8, n_real=8)
    p = workloads.make_problem(s, seed=71)
    y_head, h_head = oracle.fwd(p)
    q = dict(p)
    q["desc"] = dict(p["desc"], decay_mode="coord")
    q["A"] = np.repeat(p["A"][:, None], 8, axis=1).astype(np.float32)
    y_c, h_c = oracle.fwd(q)
    assert np.array_equal(y_head, y_c) and np.array_equal(h_head, h_c)
    r = dict(q)
    r["desc"] = dict(q["desc"], two_endpoint=True)
    r["beta"] = np.zeros_like(p["dt"]); r["gamma"] = np.ones_like(p["dt"])
    y_te, _ = oracle.fwd(r)
    assert np.array_equal(y_head, y_te)


# ---------------------------------------------------------------- P8 gradients
GRAD_PAIRS = [("x", "dx"), ("B", "dB"), ("C", "dC"), ("dt", "ddt"), ("A", "dA"),
              ("omega", "domega"), ("beta", "dbeta"), ("gamma", "dgamma"), ("D", "dD")]


@pytest.mark.parametrize("name,kw", [
    ("siso_f32", dict(seqlen=8, headdim=3, dstate=4, n_real=4, nheads=2, ngroups=2,
                      batch=2)),
    ("ssd_mimo", dict(batch=1, seqlen=7, nheads=2, ngroups=2, headdim=3, dstate=4,
                      n_real=4, rank_in=2, rank_out=2)),
    ("hybrid", dict(batch=2, seqlen=8, nheads=2, ngroups=2, headdim=3, dstate=6, n_real=2,
                    n_pairs=2, rank_in=2, rank_out=2)),
    ("hybrid", dict(batch=1, seqlen=8, nheads=4, ngroups=2, headdim=2, dstate=4, n_real=2,
                    n_pairs=1, rank_in=1, rank_out=1)),
    ("hybrid", dict(batch=1, seqlen=7, nheads=2, ngroups=2, headdim=2, dstate=8, n_real=2,
                    n_pairs=3, rank_in=2, rank_out=2, pair_rate_per_pair=True)),
    ("hybrid", dict(batch=1, seqlen=7, nheads=2, ngroups=2, headdim=2, dstate=10, n_real=4,
                    n_static=2, n_pairs=3, rank_in=2, rank_out=2, A_static_hi=3.0)),
])
def test_p8_adjoint_matches_autograd_of_quadratic_form(oracle_lib, name, kw):
    p = workloads.make_problem(small(name, **kw), seed=81, with_dy=True)
    d = p["desc"]
    rng = np.random.default_rng(82)
    h0 = rng.standard_normal((d["batch"], d["nheads"], d["dstate"], d["headdim"]))
    ins = {}
    for k, _ in GRAD_PAIRS:
        v = p.get(k)
        if v is None or (k == "omega" and d["n_pairs"] == 0):
            ins[k] = None
        else:
            ins[k] = T64(v).requires_grad_()
    h0t = T64(h0).requires_grad_()
    om = ins["omega"] if ins["omega"] is not None else torch.zeros(d["nheads"], 1,
                                                                    dtype=torch.float64)
    yq = forms.quadratic_y(d, ins["x"], ins["B"], ins["C"], ins["dt"], ins["A"], om,
                           ins["beta"], ins["gamma"], ins["D"], h0=h0t)
    (yq * T64(p["dy"])).sum().backward()
    g = oracle.bwd(p, p["dy"], h0=h0)
    for k, gk in GRAD_PAIRS:
        if ins[k] is None:
            continue
        ref = ins[k].grad.numpy()
        np.testing.assert_allclose(g[gk], ref, rtol=1e-9, atol=1e-12 * max(1, np.abs(ref).max()),
                                   err_msg=gk)
    np.testing.assert_allclose(g["dh0"], h0t.grad.numpy(), rtol=1e-9, atol=1e-13)


def test_p8_finite_differences(oracle_lib):
    s = small("hybrid", batch=1, seqlen=6, nheads=1, ngroups=1, headdim=2, dstate=4,
              n_real=2, n_pairs=1, rank_in=2, rank_out=2)
    p = workloads.make_problem(s, seed=85, with_dy=True)
    g = oracle.bwd(p, p["dy"])
    dy = p["dy"].astype(np.float64)

    def loss(q):
        y, _ = oracle.fwd(q)
        return float((y * dy).sum())

    rng = np.random.default_rng(86)
    for k, gk in [("x", "dx"), ("B", "dB"), ("C", "dC"), ("dt", "ddt"), ("beta", "dbeta"),
                  ("gamma", "dgamma")]:
        for _ in range(3):
            idx = tuple(rng.integers(0, n) for n in p[k].shape)
            # steps are taken on float32-stored inputs: use a step that survives fp32
            h = 1e-2 * max(1.0, abs(float(p[k][idx])))
            qp = dict(p); qp[k] = p[k].copy(); qp[k][idx] += np.float32(h)
            qm = dict(p); qm[k] = p[k].copy(); qm[k][idx] -= np.float32(h)
            hp = float(qp[k][idx]) - float(p[k][idx])
            hm = float(p[k][idx]) - float(qm[k][idx])
            fd = (loss(qp) - loss(qm)) / (hp + hm)
            assert abs(fd - g[gk][idx]) <= 2e-4 * max(1.0, abs(fd)), (k, idx, fd, g[gk][idx])


def test_p8_adjoint_dot_product(oracle_lib):
    # y is linear in X (for fixed B, C, dt): <dy, y(X) - y(0)> = <dX_state, X>, where
    # dX_state is the x-gradient minus the feedthrough part.
    s = small("hybrid", batch=2, seqlen=30, nheads=2, ngroups=2, headdim=4, dstate=8,
              n_real=4, n_pairs=2)
    p = workloads.make_problem(s, seed=87, with_dy=True)
    y, _ = oracle.fwd(p)
    q = dict(p); q["x"] = np.zeros_like(p["x"])
    y0, _ = oracle.fwd(q)
    g = oracle.bwd(p, p["dy"])
    lhs = float(((y - y0) * p["dy"]).sum())
    rhs = float((g["dx"] * p["x"]).sum())
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))


# ---------------------------------------------------------------- P9 state passing
def test_p9_split_run_carries_state_bitwise(oracle_lib):
    s = small("ssd_mimo", batch=2, seqlen=50, nheads=2, ngroups=2, headdim=3, dstate=4,
              n_real=4, rank_in=2, rank_out=2)
    p = workloads.make_problem(s, seed=91)
    y, hf = oracle.fwd(p)
    L1 = 23

    def part(lo, hi):
        q = dict(p)
        q["desc"] = dict(p["desc"], seqlen=hi - lo)
        for k in ("x", "B", "C", "dt"):
            q[k] = np.ascontiguousarray(p[k][:, lo:hi])
        return q

    y1, h1 = oracle.fwd(part(0, L1))
    y2, h2 = oracle.fwd(part(L1, 50), h0=h1)
    assert np.array_equal(np.concatenate([y1, y2], axis=1), y)
    assert np.array_equal(h2, hf)


def test_slice_selection_matches_full_run(oracle_lib):
    p = workloads.make_problem(small("ssd_siso", batch=3, seqlen=20, nheads=4, ngroups=4,
                                     headdim=2, dstate=4, n_real=4), seed=95)
    y, _ = oracle.fwd(p)
    ys, _ = oracle.fwd(p, slices=[(2, 1), (0, 3)])
    assert np.array_equal(ys[2, :, 1], y[2, :, 1]) and np.array_equal(ys[0, :, 3], y[0, :, 3])
    assert np.isnan(ys[1]).all()


# ---------------------------------------------------------------- P9 two-endpoint carry
def _carry_problem(seed=93, T=21):
    s = small("hybrid", batch=2, seqlen=T, nheads=2, ngroups=1, headdim=3, dstate=6, n_real=2,
              n_pairs=2, rank_in=2, rank_out=2)
    return workloads.make_problem(s, seed=seed, with_dy=True)


def _part(p, lo, hi):
    q = dict(p)
    q["desc"] = dict(p["desc"], seqlen=hi - lo)
    for k in ("x", "B", "C", "dt", "beta", "gamma", "dy"):
        q[k] = np.ascontiguousarray(p[k][:, lo:hi])
    return q


def test_p9_two_endpoint_split_run_carries_state_and_last_write_bitwise(oracle_lib):
    """A two-endpoint run split at L1 and continued with h0 = the first part's final state
    and the first part's last token (x, B) as the carried token reproduces one run bit for
    bit ("carry continuation", Blog Part 10; the initial state of Theorem 24, Part 03)."""
    p = _carry_problem()
    T, L1 = p["desc"]["seqlen"], 9
    y, hf = oracle.fwd(p)
    y1, h1 = oracle.fwd(_part(p, 0, L1))
    y2, h2 = oracle.fwd(_part(p, L1, T), h0=h1, x_prev=p["x"][:, L1 - 1], B_prev=p["B"][:, L1 - 1])
    assert np.array_equal(np.concatenate([y1, y2], axis=1), y)
    assert np.array_equal(h2, hf)
    # without the carried token the continuation misses beta_{L1} B_{L1-1} X_{L1-1}
    y2n, _ = oracle.fwd(_part(p, L1, T), h0=h1)
    assert not np.allclose(y2n, y[:, L1:])


def test_p9_split_gradients_chain_through_the_carry(oracle_lib):
    """The gradients of one run equal those of the split run chained backwards: the second
    part's dh0 enters the first part as dh_final, and its dx_prev / dB_prev add to the
    first part's last token; parameter gradients add."""
    p = _carry_problem(seed=94)
    T, L1 = p["desc"]["seqlen"], 12
    g = oracle.bwd(p, p["dy"])
    _, h1 = oracle.fwd(_part(p, 0, L1))
    p2 = _part(p, L1, T)
    g2 = oracle.bwd(p2, p2["dy"], h0=h1, x_prev=p["x"][:, L1 - 1], B_prev=p["B"][:, L1 - 1])
    p1 = _part(p, 0, L1)
    g1 = oracle.bwd(p1, p1["dy"], dh_final=g2["dh0"])
    dx1, dB1 = g1["dx"].copy(), g1["dB"].copy()
    dx1[:, L1 - 1] += g2["dx_prev"]
    dB1[:, L1 - 1] += g2["dB_prev"]
    tol = dict(rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(np.concatenate([dx1, g2["dx"]], axis=1), g["dx"], **tol)
    np.testing.assert_allclose(np.concatenate([dB1, g2["dB"]], axis=1), g["dB"], **tol)
    for k in ("dC", "ddt", "dbeta", "dgamma"):
        np.testing.assert_allclose(np.concatenate([g1[k], g2[k]], axis=1), g[k], err_msg=k, **tol)
    for k in ("dA", "domega", "dD"):
        np.testing.assert_allclose(g1[k] + g2[k], g[k], err_msg=k, **tol)
    np.testing.assert_allclose(g1["dh0"], g["dh0"], **tol)


def test_p8_carry_gradients_match_autograd_of_quadratic_form(oracle_lib):
    """dx_prev, dB_prev, dbeta_0 and the effect of dh_final, against torch autograd of the
    O(L^2) form with the carried write and the final state (loss <y, dy> + <h_final, dh_final>)."""
    p = _carry_problem(seed=95, T=7)
    d = p["desc"]
    rng = np.random.default_rng(96)
    xp = rng.standard_normal((d["batch"], d["nheads"], d["rank_in"], d["headdim"])).astype(np.float32)
    bp = rng.standard_normal((d["batch"], d["ngroups"], d["rank_in"], d["dstate"])).astype(np.float32)
    dhf = rng.standard_normal((d["batch"], d["nheads"], d["dstate"], d["headdim"]))
    h0 = rng.standard_normal((d["batch"], d["nheads"], d["dstate"], d["headdim"]))
    ins = {k: T64(p[k]).requires_grad_() for k in ("x", "B", "C", "dt", "A", "omega", "beta",
                                                    "gamma", "D")}
    xpt, bpt = T64(xp).requires_grad_(), T64(bp).requires_grad_()
    y, hf = forms.quadratic_y(d, ins["x"], ins["B"], ins["C"], ins["dt"], ins["A"], ins["omega"],
                              ins["beta"], ins["gamma"], ins["D"], h0=T64(h0), x_prev=xpt,
                              B_prev=bpt, return_state=True)
    ((y * T64(p["dy"])).sum() + (hf * T64(dhf)).sum()).backward()
    g = oracle.bwd(p, p["dy"], h0=h0, x_prev=xp, B_prev=bp, dh_final=dhf)
    yo, hfo = oracle.fwd(p, h0=h0, x_prev=xp, B_prev=bp)
    np.testing.assert_allclose(yo, y.detach().numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(hfo, hf.detach().numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["dx_prev"], xpt.grad.numpy(), rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(g["dB_prev"], bpt.grad.numpy(), rtol=1e-9, atol=1e-12)
    for k, gk in GRAD_PAIRS:
        ref = ins[k].grad.numpy()
        np.testing.assert_allclose(g[gk], ref, rtol=1e-9, atol=1e-12 * max(1, np.abs(ref).max()),
                                   err_msg=gk)


# ---------------------------------------------------------------- P10 real static rows
# Part 08 section 3 of "When a Diagonal State Is Not Enough": HybridMamba mixes real
# static, real dynamic and complex dynamic rows.  A static row's decay exp(-A_n) per token
# does not depend on the input, so a state of static rows only is a linear time-invariant
# filter of the writes.

def static_problem(T=40, N=4, P=3, seed=101, softplus=True):
    s = small("hybrid", batch=1, seqlen=T, nheads=1, ngroups=1, headdim=P, dstate=N,
              n_real=N, n_static=N, n_pairs=0, rank_in=1, rank_out=1, two_endpoint=False,
              has_D=False, dt_softplus=softplus)
    return workloads.make_problem(s, seed=seed, with_dy=True)


def test_p10_static_rows_are_first_order_iir_per_row(oracle_lib):
    # every row n is h_n <- exp(-A_n) h_n + B_n X: scipy's lfilter per row and column,
    # read out by C_t
    p = static_problem()
    y, _ = oracle.fwd(p)
    T, N, P = 40, 4, 3
    A = p["A"][0].astype(np.float64)
    Bw = p["B"][0, :, 0, 0, :].astype(np.float64)        # [T, N]
    X = p["x"][0, :, 0, 0, :].astype(np.float64)         # [T, P]
    Cr = p["C"][0, :, 0, 0, :].astype(np.float64)        # [T, N]
    ref = np.zeros((T, P))
    for n in range(N):
        a = float(np.exp(-np.float64(np.float32(A[n]))))
        hn = scipy.signal.lfilter([1.0], [1.0, -a], Bw[:, n:n + 1] * X, axis=0)  # [T, P]
        ref += Cr[:, n:n + 1] * hn
    np.testing.assert_allclose(y.reshape(T, P), ref, rtol=1e-11, atol=1e-13)


def test_p10_static_rows_ignore_the_step(oracle_lib):
    # outputs do not move with dt, and the step gradient is exactly zero
    p = static_problem()
    y, _ = oracle.fwd(p)
    q = dict(p); q["dt"] = (p["dt"] * 3.0 + 1.0).astype(np.float32)
    y2, _ = oracle.fwd(q)
    np.testing.assert_array_equal(y, y2)
    g = oracle.bwd(p, p["dy"])
    assert np.all(g["ddt"] == 0.0)


def test_p10_static_row_is_dynamic_row_at_unit_step(oracle_lib):
    # with Delta = 1 at every token (no softplus, dt = 1) a static row and a dynamic row
    # with the same rate are the same recurrence: outputs and every gradient but ddt agree
    s = small("hybrid", batch=2, seqlen=20, nheads=2, ngroups=1, headdim=3, dstate=8,
              n_real=4, n_pairs=2, rank_in=2, rank_out=2, dt_softplus=False)
    p = workloads.make_problem(s, seed=103, with_dy=True)
    p["dt"] = np.ones_like(p["dt"])
    ps = dict(p); ps["desc"] = dict(p["desc"], n_static=4)
    y0, h0 = oracle.fwd(p)
    y1, h1 = oracle.fwd(ps)
    np.testing.assert_allclose(y1, y0, rtol=1e-13, atol=1e-15)
    g0, g1 = oracle.bwd(p, p["dy"]), oracle.bwd(ps, p["dy"])
    for k in g0:
        if k == "ddt":
            continue
        np.testing.assert_allclose(g1[k], g0[k], rtol=1e-12, atol=1e-14, err_msg=k)


def test_p10_static_rows_finite_differences(oracle_lib):
    # dA of static rows and ddt (which the static rows must not feed) by central differences
    s = small("hybrid", batch=1, seqlen=9, nheads=1, ngroups=1, headdim=2, dstate=6,
              n_real=4, n_static=2, n_pairs=1, rank_in=1, rank_out=1, A_static_hi=2.0)
    p = workloads.make_problem(s, seed=105, with_dy=True)
    g = oracle.bwd(p, p["dy"])
    dy = p["dy"].astype(np.float64)

    def loss(q):
        y, _ = oracle.fwd(q)
        return float((y * dy).sum())

    for k, gk, idxs in [("A", "dA", [(0, 0), (0, 1), (0, 2)]), ("dt", "ddt", [(0, 3, 0), (0, 7, 0)])]:
        for idx in idxs:
            h = 1e-2 * max(1.0, abs(float(p[k][idx])))
            qp = dict(p); qp[k] = p[k].copy(); qp[k][idx] += np.float32(h)
            qm = dict(p); qm[k] = p[k].copy(); qm[k][idx] -= np.float32(h)
            fd = (loss(qp) - loss(qm)) / (float(qp[k][idx]) - float(qm[k][idx]))
            assert abs(fd - g[gk][idx]) <= 2e-4 * max(1.0, abs(fd)), (k, idx, fd, g[gk][idx])
