"""torch-facing wrapper: allocate outputs / saved states / workspace and call the C ABI.

Only allocation and argument marshalling happen here.  When a ``stream`` is given,
every tensor of a call (outputs, saved states, workspace) is allocated with that stream
current, so torch's caching allocator ties the memory to the stream the kernels run
on: the workspace, dropped on return, goes back to that stream's pool and is not
handed to work on another stream while the kernels may still use it.
"""
from __future__ import annotations

import contextlib

import torch

from . import _lib


def _dtype(io_dtype: str):
    return torch.bfloat16 if io_dtype == "bf16" else torch.float32


def _on(stream):
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def forward(desc_dict: dict, io_dtype: str, x, B, C, dt, A, omega=None, beta=None, gamma=None,
            D=None, save_for_backward: bool = False, chunk: int = 0, stream=None, h0=None,
            return_final_state: bool = False, x_prev=None, B_prev=None):
    """Run the forward scan.  Returns (y, saved) where saved is None unless
    ``save_for_backward``; with ``return_final_state`` returns (y, saved, h_final).
    ``h0``: optional fp32 [batch][nheads][N][P] state before token 0; ``x_prev`` /
    ``B_prev``: the token before the sequence (two-endpoint carry)."""
    desc = _lib.make_desc(desc_dict, io_dtype, chunk)
    d = desc_dict
    with _on(stream):
        y = torch.empty((d["batch"], d["seqlen"], d["nheads"], d["rank_out"], d["headdim"]),
                        dtype=_dtype(io_dtype), device=x.device)
        saved = None
        if save_for_backward:
            nbytes = _lib.saved_bytes(desc)
            saved = torch.empty(max((nbytes + 3) // 4, 1), dtype=torch.float32, device=x.device)
        wsb = _lib.workspace_bytes(desc, False)
        ws = torch.empty(wsb, dtype=torch.uint8, device=x.device) if wsb else None
        h_final = None
        if return_final_state:
            h_final = torch.empty((d["batch"], d["nheads"], d["dstate"], d["headdim"]),
                                  dtype=torch.float32, device=x.device)
        _lib.scan_fwd(desc, x, B, C, dt, A, y, omega=omega, beta=beta, gamma=gamma, D=D,
                      saved=saved, ws=ws, stream=stream, h0=h0, h_final=h_final, x_prev=x_prev,
                      B_prev=B_prev)
    if return_final_state:
        return y, saved, h_final
    return y, saved


def backward(desc_dict: dict, io_dtype: str, x, B, C, dy, dt, A, saved, omega=None, beta=None,
             gamma=None, D=None, chunk: int = 0, stream=None, want=("dA", "domega", "dbeta",
                                                                     "dgamma", "dD"),
             x_prev=None, B_prev=None, dh_final=None):
    """Run the fused reverse pass.  Returns a dict of gradient tensors (``dh0`` too
    when "dh0" is in ``want``; ``dx_prev`` and ``dB_prev`` when the carried token
    ``x_prev`` / ``B_prev`` is given).  ``dh_final``: upstream gradient of the final state."""
    desc = _lib.make_desc(desc_dict, io_dtype, chunk)
    d = desc_dict
    dev = x.device
    f32 = torch.float32
    with _on(stream):
        g = {
            "dx": torch.empty_like(x),
            "dB": torch.empty_like(B),
            "dC": torch.empty_like(C),
            "ddt": torch.empty_like(dt),
        }
        if "dA" in want:
            g["dA"] = torch.empty_like(A)
        if "domega" in want and d["n_pairs"] > 0:
            g["domega"] = torch.empty((d["nheads"], d["n_pairs"]), dtype=f32, device=dev)
        if d["two_endpoint"]:
            if "dbeta" in want:
                g["dbeta"] = torch.empty_like(dt)
            if "dgamma" in want:
                g["dgamma"] = torch.empty_like(dt)
        if d["has_D"] and "dD" in want:
            g["dD"] = torch.empty((d["nheads"],), dtype=f32, device=dev)
        if "dh0" in want:
            g["dh0"] = torch.empty((d["batch"], d["nheads"], d["dstate"], d["headdim"]),
                                   dtype=f32, device=dev)
        if x_prev is not None:
            g["dx_prev"] = torch.empty_like(x_prev)
            g["dB_prev"] = torch.empty_like(B_prev)
        wsb = _lib.workspace_bytes(desc, True)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None
        _lib.scan_bwd(desc, x, B, C, dy, dt, A, saved, g["dx"], g["dB"], g["dC"], g["ddt"],
                      omega=omega, beta=beta, gamma=gamma, D=D, dA=g.get("dA"),
                      domega=g.get("domega"), dbeta=g.get("dbeta"), dgamma=g.get("dgamma"),
                      dD=g.get("dD"), ws=ws, stream=stream, dh0=g.get("dh0"), x_prev=x_prev,
                      B_prev=B_prev, dh_final=dh_final, dx_prev=g.get("dx_prev"),
                      dB_prev=g.get("dB_prev"))
    return g


def decode_step(desc_dict: dict, io_dtype: str, x, B, C, dt, A, state, omega=None, beta=None,
                gamma=None, D=None, x_prev=None, B_prev=None, stream=None):
    """One recurrent step for every (batch, head) slice.  ``x`` [batch][nheads][R][P],
    ``B`` [batch][ngroups][R][N], ``C`` [batch][ngroups][O][N], ``dt`` [batch][nheads];
    ``state`` (fp32 [batch][nheads][N][P]) is updated in place.  Returns y
    [batch][nheads][O][P]."""
    d = dict(desc_dict, seqlen=1)
    desc = _lib.make_desc(d, io_dtype, 0)
    with _on(stream):
        y = torch.empty((d["batch"], d["nheads"], d["rank_out"], d["headdim"]),
                        dtype=_dtype(io_dtype), device=x.device)
        _lib.decode_step(desc, x, B, C, dt, A, state, y, omega=omega, beta=beta, gamma=gamma,
                         D=D, x_prev=x_prev, B_prev=B_prev, stream=stream)
    return y
