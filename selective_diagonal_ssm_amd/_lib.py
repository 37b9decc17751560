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
          -7: "SSM_ERR_HIP", -8: "SSM_ERR_SCRATCH"}
SSM_F32, SSM_BF16 = 0, 1
SSM_DECAY_HEAD, SSM_DECAY_COORD = 0, 1
SSM_F_DT_SOFTPLUS, SSM_F_TWO_ENDPOINT, SSM_F_HAS_D = 1, 2, 4

EXPORTS = ("ssm_abi_version", "ssm_status_string", "ssm_check_desc", "ssm_chunk_tokens",
           "ssm_saved_bytes", "ssm_workspace_bytes", "ssm_scan_fwd", "ssm_scan_bwd",
           "ssm_decode_step", "ssm_scratch_bytes", "ssm_scan_fwd_noalloc")


class SsmDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32),
                ("nheads", ctypes.c_int32), ("ngroups", ctypes.c_int32),
                ("headdim", ctypes.c_int32), ("dstate", ctypes.c_int32),
                ("rank_in", ctypes.c_int32), ("rank_out", ctypes.c_int32),
                ("n_real", ctypes.c_int32), ("n_pairs", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
                ("decay_mode", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("n_static", ctypes.c_int32)]


_vp = ctypes.c_void_p


class SsmFwdArgs(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("x", "B", "C", "dt", "A", "omega", "beta", "gamma", "D", "y",
                                   "saved", "h0", "h_final", "events", "x_prev", "B_prev")]


class SsmBwdArgs(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("x", "B", "C", "dy", "dt", "A", "omega", "beta", "gamma", "D",
                                   "saved", "dx", "dB", "dC", "ddt", "dA", "domega", "dbeta",
                                   "dgamma", "dD", "dh0", "events", "x_prev", "B_prev",
                                   "dh_final", "dx_prev", "dB_prev")]


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
        lib.ssm_scratch_bytes.argtypes = []
        lib.ssm_scratch_bytes.restype = ctypes.c_size_t
        lib.ssm_scan_fwd_noalloc.argtypes = [dp, ctypes.POINTER(SsmFwdArgs), _vp]
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
                   SSM_DECAY_HEAD if d["decay_mode"] == "head" else SSM_DECAY_COORD, flags,
                   d.get("n_static", 0))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# ---------------------------------------------------------------- argument checks
# The C ABI sees plain pointers, so a tensor of the wrong size, dtype or layout would be
# read or written past its end (or misread) on the device.  The wrappers below check
# every tensor against the descriptor first: the element count it implies, the dtype
# (io dtype for x, B, C, y, dy and their gradients; fp32 for the rest), contiguity and
# placement on the GPU.  Checks run before anything is enqueued.

def _io_torch_dtype(desc: SsmDesc):
    import torch
    return torch.bfloat16 if desc.io_dtype == SSM_BF16 else torch.float32


def _check(seen, name, t, numel, dtype, required=True, at_least=False):
    if t is None:
        if required and numel > 0:
            raise SsmError(-1, f"{name} is required")
        return
    n = t.numel()
    if (n < numel) if at_least else (n != numel):
        raise SsmError(-2, f"{name} has {n} elements, the descriptor needs "
                           f"{'at least ' if at_least else ''}{numel}")
    if dtype is not None and t.dtype != dtype:
        raise SsmError(-3, f"{name} is {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise SsmError(-2, f"{name} is not contiguous (the kernels read it row-major)")
    seen.append((name, t))


def _check_devices(seen):
    """After every shape check of a call: each non-empty tensor lives on the GPU."""
    for name, t in seen:
        if t.numel() > 0 and not t.is_cuda:
            raise SsmError(-1, f"{name} is not a GPU tensor")


def _na(desc: SsmDesc) -> int:
    return desc.nheads * (1 if desc.decay_mode == SSM_DECAY_HEAD else desc.n_real + desc.n_pairs)


def _check_params(seen, desc: SsmDesc, dt, A, omega, beta, gamma, D, steps: int):
    import torch
    f32 = torch.float32
    _check(seen, "dt", dt, steps, f32)
    _check(seen, "A", A, _na(desc), f32)
    _check(seen, "omega", omega, desc.nheads * desc.n_pairs, f32, required=desc.n_pairs > 0)
    te = bool(desc.flags & SSM_F_TWO_ENDPOINT)
    _check(seen, "beta", beta, steps, f32, required=te)
    _check(seen, "gamma", gamma, steps, f32, required=te)
    _check(seen, "D", D, desc.nheads, f32, required=bool(desc.flags & SSM_F_HAS_D))


def _check_scan(seen, desc: SsmDesc, x, B, C, dt, A, omega, beta, gamma, D):
    io = _io_torch_dtype(desc)
    b, L, H, G = desc.batch, desc.seqlen, desc.nheads, desc.ngroups
    _check(seen, "x", x, b * L * H * desc.rank_in * desc.headdim, io)
    _check(seen, "B", B, b * L * G * desc.rank_in * desc.dstate, io)
    _check(seen, "C", C, b * L * G * desc.rank_out * desc.dstate, io)
    _check_params(seen, desc, dt, A, omega, beta, gamma, D, b * L * H)


def _state_numel(desc: SsmDesc) -> int:
    return desc.batch * desc.nheads * desc.dstate * desc.headdim


def _check_prev(seen, desc: SsmDesc, x_prev, B_prev, names=("x_prev", "B_prev")):
    io = _io_torch_dtype(desc)
    _check(seen, names[0], x_prev, desc.batch * desc.nheads * desc.rank_in * desc.headdim, io,
           required=False)
    _check(seen, names[1], B_prev, desc.batch * desc.ngroups * desc.rank_in * desc.dstate, io,
           required=False)


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
             saved=None, ws=None, stream=None, events=None, h0=None, h_final=None, x_prev=None,
             B_prev=None) -> None:
    """Enqueue the forward scan; all tensors are caller-allocated device tensors.
    `h0` / `h_final`: optional fp32 [batch][nheads][N][P] initial / final states.
    `x_prev` / `B_prev`: the token before the sequence (two-endpoint carry).
    `events`: optional 2 torch.cuda.Event recorded around the kernel."""
    import torch
    seen = []
    _check_scan(seen, desc, x, B, C, dt, A, omega, beta, gamma, D)
    b, L, H = desc.batch, desc.seqlen, desc.nheads
    _check(seen, "y", y, b * L * H * desc.rank_out * desc.headdim, _io_torch_dtype(desc))
    if saved is not None:
        _check(seen, "saved", saved, 0, None, at_least=True)
        if saved.numel() * saved.element_size() < saved_bytes(desc):
            raise SsmError(-2, f"saved holds {saved.numel() * saved.element_size()} bytes, "
                               f"the descriptor needs {saved_bytes(desc)}")
    _check(seen, "h0", h0, _state_numel(desc), torch.float32, required=False)
    _check(seen, "h_final", h_final, _state_numel(desc), torch.float32, required=False)
    _check_prev(seen, desc, x_prev, B_prev)
    if ws is not None:
        _check(seen, "ws", ws, 0, None, at_least=True)
    _check_devices(seen)
    ev, _keep = _events(events)
    args = SsmFwdArgs(_ptr(x), _ptr(B), _ptr(C), _ptr(dt), _ptr(A), _ptr(omega), _ptr(beta),
                      _ptr(gamma), _ptr(D), _ptr(y), _ptr(saved), _ptr(h0), _ptr(h_final), ev,
                      _ptr(x_prev), _ptr(B_prev))
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    rc = load().ssm_scan_fwd(ctypes.byref(desc), ctypes.byref(args), _ptr(ws), ws_bytes,
                             _stream(stream))
    if rc != SSM_OK:
        raise SsmError(rc, "ssm_scan_fwd")


def scratch_bytes() -> int:
    """Bytes of the static scratch array that scan_fwd_noalloc uses as its workspace."""
    return load().ssm_scratch_bytes()


def scan_fwd_noalloc(desc: SsmDesc, x, B, C, dt, A, y, omega=None, beta=None, gamma=None,
                     D=None, saved=None, stream=None, h0=None, h_final=None, x_prev=None,
                     B_prev=None) -> None:
    """scan_fwd with the library's static scratch array as workspace: the call allocates
    nothing.  Raises SsmError (SSM_ERR_SCRATCH) when the problem's forward workspace
    exceeds scratch_bytes().  Calls that overlap on one GPU share the array and race."""
    import torch
    seen = []
    _check_scan(seen, desc, x, B, C, dt, A, omega, beta, gamma, D)
    b, L, H = desc.batch, desc.seqlen, desc.nheads
    _check(seen, "y", y, b * L * H * desc.rank_out * desc.headdim, _io_torch_dtype(desc))
    if saved is not None:
        _check(seen, "saved", saved, 0, None, at_least=True)
        if saved.numel() * saved.element_size() < saved_bytes(desc):
            raise SsmError(-2, f"saved holds {saved.numel() * saved.element_size()} bytes, "
                               f"the descriptor needs {saved_bytes(desc)}")
    _check(seen, "h0", h0, _state_numel(desc), torch.float32, required=False)
    _check(seen, "h_final", h_final, _state_numel(desc), torch.float32, required=False)
    _check_prev(seen, desc, x_prev, B_prev)
    _check_devices(seen)
    args = SsmFwdArgs(_ptr(x), _ptr(B), _ptr(C), _ptr(dt), _ptr(A), _ptr(omega), _ptr(beta),
                      _ptr(gamma), _ptr(D), _ptr(y), _ptr(saved), _ptr(h0), _ptr(h_final), None,
                      _ptr(x_prev), _ptr(B_prev))
    rc = load().ssm_scan_fwd_noalloc(ctypes.byref(desc), ctypes.byref(args), _stream(stream))
    if rc != SSM_OK:
        raise SsmError(rc, "ssm_scan_fwd_noalloc")


def scan_bwd(desc: SsmDesc, x, B, C, dy, dt, A, saved, dx, dB, dC, ddt, omega=None, beta=None,
             gamma=None, D=None, dA=None, domega=None, dbeta=None, dgamma=None, dD=None, ws=None,
             stream=None, events=None, dh0=None, x_prev=None, B_prev=None, dh_final=None,
             dx_prev=None, dB_prev=None) -> None:
    """Enqueue the fused reverse pass; all tensors are caller-allocated device tensors.
    `dh0`: optional fp32 [batch][nheads][N][P] gradient of the initial state.
    `x_prev` / `B_prev`: the carried token given to the forward; `dh_final`: upstream
    gradient of the final state; `dx_prev` / `dB_prev`: the carried token's gradients.
    `events`: optional 4 torch.cuda.Event recorded around the pass's three kernels."""
    import torch
    seen = []
    _check_scan(seen, desc, x, B, C, dt, A, omega, beta, gamma, D)
    io, f32 = _io_torch_dtype(desc), torch.float32
    b, L, H, G = desc.batch, desc.seqlen, desc.nheads, desc.ngroups
    _check(seen, "dy", dy, b * L * H * desc.rank_out * desc.headdim, io)
    _check(seen, "dx", dx, b * L * H * desc.rank_in * desc.headdim, io)
    _check(seen, "dB", dB, b * L * G * desc.rank_in * desc.dstate, io)
    _check(seen, "dC", dC, b * L * G * desc.rank_out * desc.dstate, io)
    _check(seen, "ddt", ddt, b * L * H, f32)
    if b * L > 0:
        _check(seen, "saved", saved, 0, None, at_least=True)
        if saved.numel() * saved.element_size() < saved_bytes(desc):
            raise SsmError(-2, f"saved holds {saved.numel() * saved.element_size()} bytes, "
                               f"the descriptor needs {saved_bytes(desc)}")
    _check(seen, "dA", dA, _na(desc), f32, required=False)
    _check(seen, "domega", domega, desc.nheads * desc.n_pairs, f32, required=False)
    _check(seen, "dbeta", dbeta, b * L * H, f32, required=False)
    _check(seen, "dgamma", dgamma, b * L * H, f32, required=False)
    _check(seen, "dD", dD, desc.nheads, f32, required=False)
    _check(seen, "dh0", dh0, _state_numel(desc), f32, required=False)
    _check_prev(seen, desc, x_prev, B_prev)
    _check_prev(seen, desc, dx_prev, dB_prev, names=("dx_prev", "dB_prev"))
    _check(seen, "dh_final", dh_final, _state_numel(desc), f32, required=False)
    if ws is not None:
        _check(seen, "ws", ws, 0, None, at_least=True)
    _check_devices(seen)
    ev, _keep = _events(events)
    args = SsmBwdArgs(_ptr(x), _ptr(B), _ptr(C), _ptr(dy), _ptr(dt), _ptr(A), _ptr(omega),
                      _ptr(beta), _ptr(gamma), _ptr(D), _ptr(saved), _ptr(dx), _ptr(dB),
                      _ptr(dC), _ptr(ddt), _ptr(dA), _ptr(domega), _ptr(dbeta), _ptr(dgamma),
                      _ptr(dD), _ptr(dh0), ev, _ptr(x_prev), _ptr(B_prev), _ptr(dh_final),
                      _ptr(dx_prev), _ptr(dB_prev))
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
    import torch
    seen = []
    io = _io_torch_dtype(desc)
    b, H, G = desc.batch, desc.nheads, desc.ngroups
    _check(seen, "x", x, b * H * desc.rank_in * desc.headdim, io)
    _check(seen, "B", B, b * G * desc.rank_in * desc.dstate, io)
    _check(seen, "C", C, b * G * desc.rank_out * desc.dstate, io)
    _check_params(seen, desc, dt, A, omega, beta, gamma, D, b * H)
    _check(seen, "x_prev", x_prev, b * H * desc.rank_in * desc.headdim, io, required=False)
    _check(seen, "B_prev", B_prev, b * G * desc.rank_in * desc.dstate, io, required=False)
    _check(seen, "state", state, _state_numel(desc), torch.float32)
    _check(seen, "y", y, b * H * desc.rank_out * desc.headdim, io)
    _check_devices(seen)
    args = SsmDecodeArgs(_ptr(x), _ptr(B), _ptr(C), _ptr(dt), _ptr(A), _ptr(omega), _ptr(beta),
                         _ptr(gamma), _ptr(D), _ptr(x_prev), _ptr(B_prev), _ptr(state), _ptr(y))
    rc = load().ssm_decode_step(ctypes.byref(desc), ctypes.byref(args), _stream(stream))
    if rc != SSM_OK:
        raise SsmError(rc, "ssm_decode_step")
