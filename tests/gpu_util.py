"""Helpers shared by the GPU parity tests: run the HIP path on a problem from
workloads.py and compare with the oracle by relative L2 (fp64)."""
import numpy as np
import torch

import selective_diagonal_ssm_amd as ssm
import workloads

BF16_TOL = 1e-2   # bf16 path: rel-L2 per tensor
F32_TOL = 1e-4    # fp32 path


def rel_l2(a, ref):
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((a - ref).ravel())
    return num / den if den > 0 else num


def tol(prob):
    return BF16_TOL if prob["dtype"] == "bf16" else F32_TOL


def rel_l2_by_position(a, ref, period, axis=1):
    """rel-L2 of the tokens at each position inside a chunk of `period` tokens
    (token index mod period along `axis`): a systematic error at one position of
    every chunk stands out here, where the whole-tensor norm would dilute it."""
    a = np.moveaxis(np.asarray(a, dtype=np.float64), axis, 0)
    ref = np.moveaxis(np.asarray(ref, dtype=np.float64), axis, 0)
    return np.array([rel_l2(a[j::period], ref[j::period]) for j in range(min(period, len(a)))])


def run_fwd(prob, chunk=0, save=False):
    chunk = chunk or prob.get("chunk", 0)  # the spec's chunk, else the library's choice
    t = workloads.to_device(prob)
    y, saved = ssm.forward(prob["desc"], prob["dtype"], t["x"], t["B"], t["C"], t["dt"], t["A"],
                           omega=t.get("omega"), beta=t.get("beta"), gamma=t.get("gamma"),
                           D=t.get("D"), save_for_backward=save, chunk=chunk)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), saved, t


def run_bwd(prob, chunk=0):
    chunk = chunk or prob.get("chunk", 0)
    y, saved, t = run_fwd(prob, chunk=chunk, save=True)
    g = ssm.backward(prob["desc"], prob["dtype"], t["x"], t["B"], t["C"], t["dy"], t["dt"],
                     t["A"], saved, omega=t.get("omega"), beta=t.get("beta"),
                     gamma=t.get("gamma"), D=t.get("D"), chunk=chunk)
    torch.cuda.synchronize()
    return y, {k: v.float().cpu().numpy().astype(np.float64) for k, v in g.items()}
