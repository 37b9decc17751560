"""ctypes binding of libssmscan.so (include/ssm_scan.h).

Argument marshalling only: every step of the scan runs in the HIP kernels.
torch supplies device memory and the current HIP stream.  If the library is
missing this module raises; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libssmscan.so")

SSM_OK = 0
STATUS = {0: "SSM_OK", -1: "SSM_ERR_NULL", -2: "SSM_ERR_SHAPE", -3: "SSM_ERR_DTYPE",
          -4: "SSM_ERR_ALIGN", -5: "SSM_ERR_UNSUPPORTED", -6: "SSM_ERR_WORKSPACE",
          -7: "SSM_ERR_HIP"}
SSM_F32, SSM_BF16 = 0, 1
SSM_DECAY_HEAD, SSM_DECAY_COORD = 0, 1
SSM_F_DT_SOFTPLUS, SSM_F_TWO_ENDPOINT, SSM_F_HAS_D = 1, 2, 4

EXPORTS = ("ssm_abi_version", "ssm_status_string", "ssm_check_desc", "ssm_chunk_tokens",
           "ssm_saved_bytes", "ssm_workspace_bytes", "ssm_scan_fwd", "ssm_scan_bwd",
           "ssm_decode_step")


class SsmDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32),
                ("nheads", ctypes.c_int32), ("ngroups", ctypes.c_int32),
                ("headdim", ctypes.c_int32), ("dstate", ctypes.c_int32),
                ("rank_in", ctypes.c_int32), ("rank_out", ctypes.c_int32),
                ("n_real", ctypes.c_int32), ("n_pairs", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
                ("decay_mode", ctypes.c_int32), ("flags", ctypes.c_uint32)]


_vp = ctypes.c_void_p


class SsmFwdArgs(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("x", "B", "C", "dt", "A", "omega", "beta", "gamma", "D", "y",
                                   "saved", "h0", "h_final", "events")]


class SsmBwdArgs(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("x", "B", "C", "dy", "dt", "A", "omega", "beta", "gamma", "D",
                                   "saved", "dx", "dB", "dC", "ddt", "dA", "domega", "dbeta",
                                   "dgamma", "dD", "dh0", "events")]


class SsmDecodeArgs(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("x", "B", "C", "dt", "A", "omega", "beta", "gamma", "D",
                                   "x_prev", "B_prev", "state", "y")]


class SsmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)}")


_lib = None


def load():
    """Load libssmscan.so (raises FileNotFoundError if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(
                f"{LIB_PATH} is missing: build it with `python -m selective_diagonal_ssm_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        dp = ctypes.POINTER(SsmDesc)
        lib.ssm_abi_version.restype = ctypes.c_int
        lib.ssm_status_string.argtypes = [ctypes.c_int]
        lib.ssm_status_string.restype = ctypes.c_char_p
        lib.ssm_check_desc.argtypes = [dp]
        lib.ssm_chunk_tokens.argtypes = [dp]
        lib.ssm_saved_bytes.argtypes = [dp]
        lib.ssm_saved_bytes.restype = ctypes.c_size_t
        lib.ssm_workspace_bytes.argtypes = [dp, ctypes.c_int]
        lib.ssm_workspace_bytes.restype = ctypes.c_size_t
        lib.ssm_scan_fwd.argtypes = [dp, ctypes.POINTER(SsmFwdArgs), _vp, ctypes.c_size_t, _vp]
        lib.ssm_scan_bwd.argtypes = [dp, ctypes.POINTER(SsmBwdArgs), _vp, ctypes.c_size_t, _vp]
        lib.ssm_decode_step.argtypes = [dp, ctypes.POINTER(SsmDecodeArgs), _vp]
        _lib = lib
    return _lib


def make_desc(d: dict, io_dtype: str, chunk: int = 0) -> SsmDesc:
    """Descriptor from a shape/flag dict (keys as in workloads.DESC_KEYS)."""
    flags = ((SSM_F_DT_SOFTPLUS if d["dt_softplus"] else 0)
             | (SSM_F_TWO_ENDPOINT if d["two_endpoint"] else 0)
             | (SSM_F_HAS_D if d["has_D"] else 0))
    return SsmDesc(d["batch"], d["seqlen"], d["nheads"], d["ngroups"], d["headdim"], d["dstate"],
                   d["rank_in"], d["rank_out"], d["n_real"], d["n_pairs"], chunk,
                   SSM_BF16 if io_dtype == "bf16" else SSM_F32,
                   SSM_DECAY_HEAD if d["decay_mode"] == "head" else SSM_DECAY_COORD, flags)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def check_desc(desc: SsmDesc) -> int:
    return load().ssm_check_desc(ctypes.byref(desc))


def chunk_tokens(desc: SsmDesc) -> int:
    return load().ssm_chunk_tokens(ctypes.byref(desc))


def saved_bytes(desc: SsmDesc) -> int:
    return load().ssm_saved_bytes(ctypes.byref(desc))


def workspace_bytes(desc: SsmDesc, for_backward: bool) -> int:
    return load().ssm_workspace_bytes(ctypes.byref(desc), int(for_backward))


def _events(events):
    """ctypes array of hipEvent_t handles from torch.cuda.Event objects (recorded once
    beforehand so that the handles exist; a None entry is not recorded), or None."""
    if not events:
        return None, None
    arr = (ctypes.c_void_p * len(events))(
        *[ctypes.c_void_p(None if e is None else e.cuda_event) for e in events])
    return ctypes.cast(arr, ctypes.c_void_p), arr


def scan_fwd(desc: SsmDesc, x, B, C, dt, A, y, omega=None, beta=None, gamma=None, D=None,
             saved=None, ws=None, stream=None, events=None, h0=None, h_final=None) -> None:
    """Enqueue the forward scan; all tensors are caller-allocated device tensors.
    `h0` / `h_final`: optional fp32 [batch][nheads][N][P] initial / final states.
    `events`: optional 2 torch.cuda.Event recorded around the kernel."""
    ev, _keep = _events(events)
    args = SsmFwdArgs(_ptr(x), _ptr(B), _ptr(C), _ptr(dt), _ptr(A), _ptr(omega), _ptr(beta),
                      _ptr(gamma), _ptr(D), _ptr(y), _ptr(saved), _ptr(h0), _ptr(h_final), ev)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    rc = load().ssm_scan_fwd(ctypes.byref(desc), ctypes.byref(args), _ptr(ws), ws_bytes,
                             _stream(stream))
    if rc != SSM_OK:
        raise SsmError(rc, "ssm_scan_fwd")


def scan_bwd(desc: SsmDesc, x, B, C, dy, dt, A, saved, dx, dB, dC, ddt, omega=None, beta=None,
             gamma=None, D=None, dA=None, domega=None, dbeta=None, dgamma=None, dD=None, ws=None,
             stream=None, events=None, dh0=None) -> None:
    """Enqueue the fused reverse pass; all tensors are caller-allocated device tensors.
    `dh0`: optional fp32 [batch][nheads][N][P] gradient of the initial state.
    `events`: optional 4 torch.cuda.Event recorded around the pass's three kernels."""
    ev, _keep = _events(events)
    args = SsmBwdArgs(_ptr(x), _ptr(B), _ptr(C), _ptr(dy), _ptr(dt), _ptr(A), _ptr(omega),
                      _ptr(beta), _ptr(gamma), _ptr(D), _ptr(saved), _ptr(dx), _ptr(dB),
                      _ptr(dC), _ptr(ddt), _ptr(dA), _ptr(domega), _ptr(dbeta), _ptr(dgamma),
                      _ptr(dD), _ptr(dh0), ev)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    rc = load().ssm_scan_bwd(ctypes.byref(desc), ctypes.byref(args), _ptr(ws), ws_bytes,
                             _stream(stream))
    if rc != SSM_OK:
        raise SsmError(rc, "ssm_scan_bwd")


def decode_step(desc: SsmDesc, x, B, C, dt, A, state, y, omega=None, beta=None, gamma=None,
                D=None, x_prev=None, B_prev=None, stream=None) -> None:
    """Enqueue one recurrent step (descriptor with seqlen 1): updates the fp32
    [batch][nheads][N][P] `state` in place and writes y.  `x_prev` / `B_prev`: the
    previous token's x and B for two-endpoint writes (None at the first token)."""
    args = SsmDecodeArgs(_ptr(x), _ptr(B), _ptr(C), _ptr(dt), _ptr(A), _ptr(omega), _ptr(beta),
                         _ptr(gamma), _ptr(D), _ptr(x_prev), _ptr(B_prev), _ptr(state), _ptr(y))
    rc = load().ssm_decode_step(ctypes.byref(desc), ctypes.byref(args), _stream(stream))
    if rc != SSM_OK:
        raise SsmError(rc, "ssm_decode_step")
