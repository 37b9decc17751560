"""Independent small-size forms that pin the recurrence oracle (TEST INFRASTRUCTURE ONLY).

None of these calls the C oracle; each is a separate derivation from the pages:

* ``quadratic_y`` -- the O(L^2) masked-linear-attention form.  "When a Diagonal
  State Is Not Enough" (sungsoo.github.io), Part 03, Theorem 24 identifies the
  state-mediated kernel with unnormalized linear attention under a
  multiplicative mask, including the initial state and the direct
  feedthrough:  y_t = sum_{s<=t} C_t^T M_{t,s} X_s + C_t^T Phi_{t,-1} h0 + D X_t,
  where every transfer Phi_{t,s} = A_t ... A_{s+1} is rebuilt here as an
  explicit product of full N x N transition matrices.  Written in torch fp64
  so that autograd yields an independently derived gradient of every input.
* ``complex_y`` -- the complex-diagonal form of the rotating pairs (Part 03,
  Theorem 8: a commuting family with non-real eigenvalues diagonalizes over C,
  not over R): each pair is one complex mode z <- rho e^{i theta} z + w, read
  out as Re(conj(c) z).
* ``transfer`` -- the local transfer C_t Phi_{t,s} B_s of Theorem 21 (Part 01 and
  Part 08.2), assembled from explicit matrices.
"""
from __future__ import annotations

import numpy as np
import torch


def _t(a):
    return torch.as_tensor(np.asarray(a, dtype=np.float64))


def transition_matrices(desc: dict, dt, A, omega):
    """Full N x N transition A_t for every (b, t, h): tensor [b, T, H, N, N].
    Real static rows (Part 08 section 3 of the same page: HybridMamba's real static,
    real dynamic and complex dynamic rows) decay by exp(-A) per token, whatever Delta."""
    b, T, H, N = desc["batch"], desc["seqlen"], desc["nheads"], desc["dstate"]
    nr, npairs = desc["n_real"], desc["n_pairs"]
    delta = torch.nn.functional.softplus(dt) if desc["dt_softplus"] else dt
    Am = torch.zeros(b, T, H, N, N, dtype=torch.float64)
    for h in range(H):
        if desc["decay_mode"] == "head":
            rates = [A[h]] * N
            prates = []
        else:
            rates = [A[h, n] for n in range(nr)]
            prates = [A[h, nr + k] for k in range(npairs)]
        for n in range(nr):
            # a static row (the first n_static real rows) takes a unit step at every token
            step = 1.0 if n < desc.get("n_static", 0) else delta[:, :, h]
            Am[:, :, h, n, n] = torch.exp(-step * rates[n])
        for k in range(npairs):
            i, j = nr + 2 * k, nr + 2 * k + 1
            rho = torch.exp(-delta[:, :, h] * prates[k])
            th = delta[:, :, h] * omega[h, k]
            Am[:, :, h, i, i] = rho * torch.cos(th)
            Am[:, :, h, i, j] = -rho * torch.sin(th)
            Am[:, :, h, j, i] = rho * torch.sin(th)
            Am[:, :, h, j, j] = rho * torch.cos(th)
    return Am


def quadratic_y(desc: dict, x, B, C, dt, A, omega=None, beta=None, gamma=None, D=None, h0=None,
                x_prev=None, B_prev=None, return_state=False):
    """O(L^2) form of Theorem 24 with explicit transfer products (torch fp64 tensors in/out).
    `x_prev` [b][H][R][P] / `B_prev` [b][G][R][N]: the token before the sequence, whose
    two-endpoint write beta_0 B_prev X_prev enters at token 0 and reaches token t through
    Phi_{t,0}.  With `return_state`, returns (y, h_final), h_final [b][H][N][P] being the
    state after the last token summed the same way."""
    b, T, H, G = desc["batch"], desc["seqlen"], desc["nheads"], desc["ngroups"]
    P, N, R, O = desc["headdim"], desc["dstate"], desc["rank_in"], desc["rank_out"]
    if omega is None:
        omega = torch.zeros(H, max(desc["n_pairs"], 1), dtype=torch.float64)
    Am = transition_matrices(desc, dt, A, omega)
    eye = torch.eye(N, dtype=torch.float64)
    ys = []
    finals = []  # h_{T-1} per (batch, head), in that order
    for bb in range(b):
        yb = []
        for t in range(T):
            yh = []
            for h in range(H):
                g = h // (H // G)
                # Phi[s] = A_t ... A_{s+1} for s = t, t-1, ..., -1
                phis = {t: eye}
                cur = eye
                for s in range(t - 1, -2, -1):
                    cur = cur @ Am[bb, s + 1, h]
                    phis[s] = cur
                acc = torch.zeros(N, P, dtype=torch.float64)
                for s in range(0, t + 1):
                    w = B[bb, s, g].T @ x[bb, s, h]  # N x P, the write B_s X_s
                    gm = gamma[bb, s, h] if desc["two_endpoint"] else 1.0
                    acc = acc + gm * (phis[s] @ w)
                    if desc["two_endpoint"] and s + 1 <= t:
                        acc = acc + beta[bb, s + 1, h] * (phis[s + 1] @ w)
                if h0 is not None:
                    acc = acc + phis[-1] @ h0[bb, h]
                if desc["two_endpoint"] and x_prev is not None:
                    acc = acc + beta[bb, 0, h] * (phis[0] @ (B_prev[bb, g].T @ x_prev[bb, h]))
                if return_state and t == T - 1:
                    finals.append(acc)
                yt = C[bb, t, g] @ acc  # O x P
                if desc["has_D"]:
                    yt = yt + D[h] * x[bb, t, h]
                yh.append(yt)
            yb.append(torch.stack(yh))
        ys.append(torch.stack(yb))
    y = torch.stack(ys)  # [b, T, H, O, P]
    if return_state:
        return y, torch.stack(finals).reshape(b, H, N, P)
    return y


def complex_y(desc: dict, x, B, C, dt, A, omega, beta=None, gamma=None, D=None):
    """Complex-diagonal recurrence (numpy complex128).  Real rows stay real
    scalar modes; pair k is the complex mode z = h_{2k} + i h_{2k+1}."""
    b, T, H, G = desc["batch"], desc["seqlen"], desc["nheads"], desc["ngroups"]
    P, N, R, O = desc["headdim"], desc["dstate"], desc["rank_in"], desc["rank_out"]
    nr, npairs = desc["n_real"], desc["n_pairs"]
    x, B, C, dt, A, omega = (np.asarray(a, dtype=np.float64) for a in (x, B, C, dt, A, omega))
    delta = np.logaddexp(0.0, dt) if desc["dt_softplus"] else dt
    y = np.zeros((b, T, H, O, P))
    for bb in range(b):
        for h in range(H):
            g = h // (H // G)
            hr = np.zeros((nr, P))
            z = np.zeros((npairs, P), dtype=np.complex128)
            prev = None
            for t in range(T):
                d = delta[bb, t, h]
                # static rows (the first n_static) take a unit step whatever Delta is
                ar = np.exp(-np.where(np.arange(nr) < desc.get("n_static", 0), 1.0, d) * A[h, :nr])
                lam = np.exp(-d * A[h, nr:nr + npairs] + 1j * d * omega[h, :npairs])
                w = B[bb, t, g].T @ x[bb, t, h]  # N x P
                gm = gamma[bb, t, h] if desc["two_endpoint"] else 1.0
                wt = gm * w
                if desc["two_endpoint"] and prev is not None:
                    wt = wt + beta[bb, t, h] * prev
                prev = w
                hr = ar[:, None] * hr + wt[:nr]
                wz = wt[nr::2][:npairs] + 1j * wt[nr + 1::2][:npairs]
                z = lam[:, None] * z + wz
                for o in range(O):
                    c = C[bb, t, g, o]
                    cz = c[nr::2][:npairs] + 1j * c[nr + 1::2][:npairs]
                    y[bb, t, h, o] = c[:nr] @ hr + np.real(np.conj(cz) @ z)
                if desc["has_D"]:
                    y[bb, t, h] += D[h] * x[bb, t, h]
    return y


def transfer(desc: dict, B, C, dt, A, omega, beta, gamma, bb, h, t, s):
    """J_{ts} = C_t^T (gamma_s Phi_{t,s} + beta_{s+1} Phi_{t,s+1}) B_s  (O x R), s <= t."""
    g = h // (desc["nheads"] // desc["ngroups"])
    N = desc["dstate"]
    Am = transition_matrices(desc, _t(dt), _t(A), _t(omega))
    phi_s = torch.eye(N, dtype=torch.float64)
    for r in range(t, s, -1):
        phi_s = phi_s @ Am[bb, r, h]
    gm = float(gamma[bb, s, h]) if desc["two_endpoint"] else 1.0
    M = gm * phi_s
    if desc["two_endpoint"] and s + 1 <= t:
        phi_s1 = torch.eye(N, dtype=torch.float64)
        for r in range(t, s + 1, -1):
            phi_s1 = phi_s1 @ Am[bb, r, h]
        M = M + float(beta[bb, s + 1, h]) * phi_s1
    return (_t(C[bb, t, g]) @ M @ _t(B[bb, s, g]).T).numpy()
