"""Seeded synthetic inputs for the state-mediated SSM kernel.

This module is shared by the oracle tests and the GPU path (tests, bench).  It
holds none of the method's arithmetic: it only draws random numbers in a fixed
order, rounds the values that are stored as bfloat16 (round to nearest even,
from fp32) and describes shapes.  Kernels receive the raw dt and apply
softplus themselves (flag ``dt_softplus``).

Workloads (names follow the method's own vocabulary):

=====================  =============================================================
siso_f32               SISO real scan, fp32: b=1, L=256, H=1, P=16, N=16, R=1, head
                       decay A=1, dt ~ N(0,1)-0.5 (softplus in kernel),
                       x, B, C ~ N(0,1)/sqrt(N), D=0
ssd_siso               Mamba-2-style SSD SISO, bf16: b=8, L=2048, H=24, P=64, N=128,
                       R=1, head decay, dt_raw ~ N(-2, 0.5), A_h ~ U[1,16],
                       x, B, C ~ N(0,1), D ~ N(0,1)
ssd_mimo               SSD-MIMO, bf16: b=8, L=4096, H=16, P=64, N=64, R=O=4, head
                       decay, dt/A as ssd_siso, x, B, C ~ N(0,1)/sqrt(N R), D ~ N(0,1)
hybrid                 HybridMamba fwd, bf16: b=4, L=8192, H=32, P=64, N=64 = 32 real
                       rows (per-coordinate rates U[1,16]) + 16 rotating pairs (rate
                       A_h ~ U[1,16] shared by the head's pairs, omega ~ U[0, pi]),
                       two-endpoint write with beta, gamma ~ sigmoid(N(0,1)), R=O=2,
                       x, B, C ~ N(0,1)/sqrt(N R), D ~ N(0,1)
hybrid_r1              hybrid at R=O=1 (two-endpoint SISO interface)
hybrid_bwd             hybrid at b=2, L=16384, fwd + bwd, dy ~ N(0,1)
ssd_mimo_bwd           ssd_mimo at b=2, L=16384, fwd + bwd, dy ~ N(0,1)
=====================  =============================================================

Draw order (numpy PCG64, ``default_rng(seed)``): dt, A, omega, beta, gamma, D,
x, B, C, dy.

Optional spec keys (absent from the workloads above, so their draws are unchanged):

``pair_rate_per_pair``  draw the rotating pairs' decay rates per (head, pair) instead of
                        one per head (the pairs of a head then decay at different rates)
``n_static``            the first n_static real rows are static (per-row decay only): their
                        decay exp(-A) per token does not depend on the step; their rates are
                        drawn ~ U[A_static_lo, A_static_hi] (default U[0.01, 1]) from a third
                        generator, ``default_rng([seed, 2])``, so the other draws do not move
``dt_spike_prob``       probability (a float, or a list with one entry per head) that a
                        token's raw step is replaced by a spike ~ N(dt_spike_mean,
                        dt_spike_std): steps large enough to wipe a state row within a
                        few tokens.  Spikes come from a second generator,
                        ``default_rng([seed, 1])``, so the other draws do not move.
"""
from __future__ import annotations

import copy
import math

import numpy as np

WORKLOADS = {
    "siso_f32": dict(batch=1, seqlen=256, nheads=1, ngroups=1, headdim=16, dstate=16,
                     rank_in=1, rank_out=1, n_real=16, n_pairs=0, decay_mode="head",
                     dt_softplus=True, two_endpoint=False, has_D=False, dtype="f32",
                     dt_mean=-0.5, dt_std=1.0, A_fixed=1.0, xbc_scale=1 / math.sqrt(16),
                     backward=False),
    "ssd_siso": dict(batch=8, seqlen=2048, nheads=24, ngroups=24, headdim=64, dstate=128,
                     rank_in=1, rank_out=1, n_real=128, n_pairs=0, decay_mode="head",
                     dt_softplus=True, two_endpoint=False, has_D=True, dtype="bf16",
                     dt_mean=-2.0, dt_std=0.5, A_lo=1.0, A_hi=16.0, xbc_scale=1.0,
                     backward=False, chunk=64),
    "ssd_mimo": dict(batch=8, seqlen=4096, nheads=16, ngroups=16, headdim=64, dstate=64,
                     rank_in=4, rank_out=4, n_real=64, n_pairs=0, decay_mode="head",
                     dt_softplus=True, two_endpoint=False, has_D=True, dtype="bf16",
                     dt_mean=-2.0, dt_std=0.5, A_lo=1.0, A_hi=16.0,
                     xbc_scale=1 / math.sqrt(64 * 4), backward=False),
    "hybrid": dict(batch=4, seqlen=8192, nheads=32, ngroups=32, headdim=64, dstate=64,
                   rank_in=2, rank_out=2, n_real=32, n_pairs=16, decay_mode="coord",
                   dt_softplus=True, two_endpoint=True, has_D=True, dtype="bf16",
                   dt_mean=-2.0, dt_std=0.5, A_lo=1.0, A_hi=16.0,
                   xbc_scale=1 / math.sqrt(64 * 2), backward=False),
}
WORKLOADS["hybrid_r1"] = dict(WORKLOADS["hybrid"], rank_in=1, rank_out=1,
                              xbc_scale=1 / math.sqrt(64))
WORKLOADS["hybrid_bwd"] = dict(WORKLOADS["hybrid"], batch=2, seqlen=16384, backward=True)
WORKLOADS["ssd_mimo_bwd"] = dict(WORKLOADS["ssd_mimo"], batch=2, seqlen=16384, backward=True)

DESC_KEYS = ("batch", "seqlen", "nheads", "ngroups", "headdim", "dstate", "rank_in",
             "rank_out", "n_real", "n_pairs", "decay_mode", "dt_softplus", "two_endpoint",
             "has_D")


def round_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bfloat16 value (ties to even), returned as fp32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32)


def spec(name: str, **overrides) -> dict:
    """Workload spec with optional shape overrides (e.g. a smaller seqlen)."""
    s = copy.deepcopy(WORKLOADS[name])
    s.update(overrides)
    return s


def make_problem(spec_or_name, seed: int = 0, with_dy: bool | None = None) -> dict:
    """Draw one problem.  Returns a dict with ``desc`` (shape/flags), ``dtype``
    and float32 numpy arrays x, B, C, dt, A, omega, beta, gamma, D (and dy).
    Arrays stored as bf16 on the GPU are already rounded to bf16 values."""
    s = WORKLOADS[spec_or_name] if isinstance(spec_or_name, str) else spec_or_name
    rng = np.random.default_rng(seed)
    b, T, H, G = s["batch"], s["seqlen"], s["nheads"], s["ngroups"]
    P, N, R, O = s["headdim"], s["dstate"], s["rank_in"], s["rank_out"]
    nr, npairs = s["n_real"], s["n_pairs"]
    f32 = np.float32
    dt = (rng.standard_normal((b, T, H), dtype=f32) * f32(s["dt_std"]) + f32(s["dt_mean"]))
    if s["decay_mode"] == "head":
        if "A_fixed" in s:
            A = np.full((H,), s["A_fixed"], dtype=f32)
        else:
            A = rng.uniform(s["A_lo"], s["A_hi"], size=(H,)).astype(f32)
    else:
        real = rng.uniform(s["A_lo"], s["A_hi"], size=(H, nr)).astype(f32)
        if s.get("pair_rate_per_pair", False):
            pair_rate = rng.uniform(s["A_lo"], s["A_hi"], size=(H, npairs)).astype(f32)
        else:
            pair_rate = np.repeat(rng.uniform(s["A_lo"], s["A_hi"], size=(H,)).astype(f32)[:, None],
                                  npairs, axis=1)
        A = np.concatenate([real, pair_rate], axis=1)
        A = np.ascontiguousarray(A, dtype=f32)
    omega = (rng.uniform(0.0, math.pi, size=(H, npairs)).astype(f32) if npairs
             else np.zeros((H, 0), dtype=f32))
    if s["two_endpoint"]:
        beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((b, T, H))))).astype(f32)
        gamma = (1.0 / (1.0 + np.exp(-rng.standard_normal((b, T, H))))).astype(f32)
    else:
        beta = gamma = None
    D = rng.standard_normal((H,)).astype(f32) if s["has_D"] else None
    sc = f32(s["xbc_scale"])
    x = rng.standard_normal((b, T, H, R, P), dtype=f32) * sc
    B = rng.standard_normal((b, T, G, R, N), dtype=f32) * sc
    C = rng.standard_normal((b, T, G, O, N), dtype=f32) * sc
    want_dy = s.get("backward", False) if with_dy is None else with_dy
    dy = rng.standard_normal((b, T, H, O, P), dtype=f32) if want_dy else None
    spike = s.get("dt_spike_prob", 0.0)
    if np.any(np.asarray(spike) > 0):
        r2 = np.random.default_rng([seed, 1])
        prob_h = np.broadcast_to(np.asarray(spike, dtype=np.float64), (H,))
        hit = r2.random((b, T, H)) < prob_h
        val = (r2.standard_normal((b, T, H), dtype=f32) * f32(s.get("dt_spike_std", 0.5))
               + f32(s.get("dt_spike_mean", 2.0)))
        dt = np.where(hit, val, dt).astype(f32)
    if s["dtype"] == "bf16":
        x, B, C = round_bf16(x), round_bf16(B), round_bf16(C)
        dy = round_bf16(dy) if dy is not None else None
    ns = s.get("n_static", 0)
    if ns:
        r3 = np.random.default_rng([seed, 2])
        A[:, :ns] = r3.uniform(s.get("A_static_lo", 0.01), s.get("A_static_hi", 1.0),
                               size=(H, ns)).astype(f32)
    desc = {k: s[k] for k in DESC_KEYS}
    desc["n_static"] = ns
    prob = dict(desc=desc, dtype=s["dtype"], chunk=s.get("chunk", 0),
                x=x, B=B, C=C, dt=dt, A=A, omega=omega, beta=beta, gamma=gamma, D=D, dy=dy)
    return prob


def make_state(desc: dict, seed: int = 0, scale: float = 1.0) -> np.ndarray:
    """A seeded initial state h0, fp32 [batch][nheads][dstate][headdim] ~ N(0, scale^2)."""
    rng = np.random.default_rng(seed)
    shape = (desc["batch"], desc["nheads"], desc["dstate"], desc["headdim"])
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)).astype(np.float32)


def to_device(prob: dict, device="cuda"):
    """Copy a problem's arrays to torch tensors on `device` (x, B, C, dy in the
    io dtype; the rest fp32)."""
    import torch

    io = torch.bfloat16 if prob["dtype"] == "bf16" else torch.float32
    out = {}
    for k in ("x", "B", "C", "dy"):
        if prob.get(k) is not None:
            out[k] = torch.from_numpy(prob[k]).to(device=device).to(io).contiguous()
    for k in ("dt", "A", "omega", "beta", "gamma", "D"):
        v = prob.get(k)
        if v is not None and (k != "omega" or v.size):
            out[k] = torch.from_numpy(np.ascontiguousarray(v)).to(device=device).contiguous()
    return out
