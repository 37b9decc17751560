"""ctypes front-end of the fp64 C oracle (TEST INFRASTRUCTURE ONLY).

The C source (``ssm_oracle.c``) is the plain sequential recurrence of
"When a Diagonal State Is Not Enough" (sungsoo.github.io), Part 01 / Part 03,
with complex modes as rotating 2x2 pairs (Part 03, Theorem 8) and SSD-MIMO /
HybridMamba writes (Parts 03 and 08.3).  This module only marshals numpy
arrays; it performs none of the method's arithmetic itself, except the fixed
order summation of per-slice parameter-gradient partials.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def lib_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile ssm_oracle.c with gcc (-O2, OpenMP, fp64, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "batch", "seqlen", "nheads", "ngroups", "headdim", "dstate", "rank_in", "rank_out",
        "n_real", "n_pairs", "decay_mode", "dt_softplus", "two_endpoint", "has_D", "n_static")]


@dataclass
class OracleDesc:
    batch: int
    seqlen: int
    nheads: int
    ngroups: int
    headdim: int
    dstate: int
    rank_in: int
    rank_out: int
    n_real: int
    n_pairs: int
    decay_mode: str  # "head" | "coord"
    dt_softplus: bool
    two_endpoint: bool
    has_D: bool
    n_static: int = 0  # the first n_static real rows decay by exp(-A) per token

    def c(self) -> _Desc:
        return _Desc(self.batch, self.seqlen, self.nheads, self.ngroups, self.headdim,
                     self.dstate, self.rank_in, self.rank_out, self.n_real, self.n_pairs,
                     0 if self.decay_mode == "head" else 1, int(self.dt_softplus),
                     int(self.two_endpoint), int(self.has_D), int(self.n_static))

    @classmethod
    def from_dict(cls, d: dict) -> "OracleDesc":
        return cls(**{k: d[k] for k in cls.__dataclass_fields__ if k in d})


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        fp = ctypes.POINTER(ctypes.c_float)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int)
        lib.oracle_fwd.argtypes = ([ctypes.POINTER(_Desc)] + [fp] * 9 + [dp, fp, fp, dp, dp, ip,
                                                                           ctypes.c_int])
        lib.oracle_fwd.restype = ctypes.c_int
        lib.oracle_bwd.argtypes = ([ctypes.POINTER(_Desc)] + [fp] * 9 + [dp, fp, fp, fp, dp]
                                   + [dp] * 12 + [ip, ctypes.c_int])
        lib.oracle_bwd.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f32(a):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _fptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_float)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _dptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _slices(desc: OracleDesc, slices):
    if slices is None:
        slices = [(b, h) for b in range(desc.batch) for h in range(desc.nheads)]
    arr = np.ascontiguousarray(np.asarray(slices, dtype=np.int32).reshape(-1, 2))
    return arr


def _inputs(prob):
    keys = ("x", "B", "C", "dt", "A", "omega", "beta", "gamma", "D")
    return [_f32(prob.get(k)) for k in keys]


def fwd(prob: dict, slices=None, h0=None, x_prev=None, B_prev=None):
    """Run the oracle forward.  Returns (y, h_final) as float64 arrays; entries
    of slices that were not requested are NaN.  `x_prev` [b][h][R][P] and `B_prev`
    [b][g][R][N]: the token before the sequence (two-endpoint carry)."""
    desc = OracleDesc.from_dict(prob["desc"])
    lib = load()
    x, B, C, dt, A, om, be, ga, D = _inputs(prob)
    b, T, H, P, N, O = desc.batch, desc.seqlen, desc.nheads, desc.headdim, desc.dstate, desc.rank_out
    y = np.full((b, T, H, O, P), np.nan, dtype=np.float64)
    hf = np.full((b, H, N, P), np.nan, dtype=np.float64)
    h0 = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64)
    sl = _slices(desc, slices)
    dc = desc.c()
    xp, bp = _f32(x_prev), _f32(B_prev)
    rc = lib.oracle_fwd(ctypes.byref(dc), _fptr(x), _fptr(B), _fptr(C), _fptr(dt), _fptr(A),
                        _fptr(om), _fptr(be), _fptr(ga), _fptr(D), _dptr(h0), _fptr(xp),
                        _fptr(bp), _dptr(y), _dptr(hf),
                        sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), len(sl))
    if rc:
        raise ValueError(f"oracle_fwd rejected the descriptor (rc={rc})")
    return y, hf


def bwd(prob: dict, dy, slices=None, h0=None, x_prev=None, B_prev=None, dh_final=None):
    """Run the oracle reverse mode.  Returns a dict with dx, dB, dC, ddt, dA,
    domega, dbeta, dgamma, dD, dh0, dx_prev, dB_prev (float64).  Per-token gradients of
    slices that were not requested are NaN (dB/dC: zero); dA/domega/dD sum over the
    requested slices only.  `x_prev` / `B_prev`: the token before the sequence (its
    gradients come back as dx_prev / dB_prev); `dh_final`: upstream gradient of the final
    state [b][h][N][P]."""
    desc = OracleDesc.from_dict(prob["desc"])
    lib = load()
    x, B, C, dt, A, om, be, ga, D = _inputs(prob)
    dy = _f32(dy)
    b, T, H, G = desc.batch, desc.seqlen, desc.nheads, desc.ngroups
    P, N, R, O = desc.headdim, desc.dstate, desc.rank_in, desc.rank_out
    nA = 1 if desc.decay_mode == "head" else desc.n_real + desc.n_pairs
    npairs = desc.n_pairs
    sl = _slices(desc, slices)
    ns = len(sl)
    out = {
        "dx": np.full((b, T, H, R, P), np.nan),
        "dB": np.zeros((b, T, G, R, N)) if G != H else np.full((b, T, G, R, N), np.nan),
        "dC": np.zeros((b, T, G, O, N)) if G != H else np.full((b, T, G, O, N), np.nan),
        "ddt": np.full((b, T, H), np.nan),
        "dbeta": np.full((b, T, H), np.nan),
        "dgamma": np.full((b, T, H), np.nan),
        "dh0": np.full((b, H, N, P), np.nan),
        "dx_prev": np.full((b, H, R, P), np.nan),
        "dB_prev": np.zeros((b, G, R, N)),
    }
    dA_s = np.zeros((ns, nA))
    dw_s = np.zeros((ns, max(npairs, 1)))
    dD_s = np.zeros((ns,))
    h0 = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64)
    dc = desc.c()
    xp, bp = _f32(x_prev), _f32(B_prev)
    dhf = None if dh_final is None else np.ascontiguousarray(dh_final, dtype=np.float64)
    rc = lib.oracle_bwd(ctypes.byref(dc), _fptr(x), _fptr(B), _fptr(C), _fptr(dt), _fptr(A),
                        _fptr(om), _fptr(be), _fptr(ga), _fptr(D), _dptr(h0), _fptr(xp),
                        _fptr(bp), _fptr(dy), _dptr(dhf),
                        _dptr(out["dx"]), _dptr(out["dB"]), _dptr(out["dC"]), _dptr(out["ddt"]),
                        _dptr(dA_s), _dptr(dw_s), _dptr(out["dbeta"]), _dptr(out["dgamma"]),
                        _dptr(dD_s), _dptr(out["dh0"]), _dptr(out["dx_prev"]),
                        _dptr(out["dB_prev"]),
                        sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), ns)
    if rc:
        raise ValueError(f"oracle_bwd rejected the descriptor (rc={rc})")
    # fixed-order reduction of per-slice partials into per-head parameter grads
    dA = np.zeros((H, nA))
    dw = np.zeros((H, max(npairs, 1)))
    dD = np.zeros((H,))
    for i, (_, h) in enumerate(sl):
        dA[h] += dA_s[i]
        dw[h] += dw_s[i]
        dD[h] += dD_s[i]
    out["dA"] = dA[:, 0] if desc.decay_mode == "head" else dA
    out["domega"] = dw[:, :npairs]
    out["dD"] = dD
    return out
