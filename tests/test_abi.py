"""CPU checks of the C-ABI library: it loads, exports every symbol the header
declares, and rejects bad descriptors / pointers before any GPU call."""
import ctypes
import os
import re

import pytest

import selective_diagonal_ssm_amd as ssm
from selective_diagonal_ssm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "ssm_scan.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ssm_\w+)\s*\(", src, re.M)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    names = header_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings():
    lib = ssm.load()
    assert lib.ssm_abi_version() == 6
    for s in range(0, -9, -1):
        assert lib.ssm_status_string(s)


def base_desc(**kw):
    d = dict(batch=2, seqlen=100, nheads=4, ngroups=4, headdim=64, dstate=64, rank_in=1,
             rank_out=1, n_real=64, n_pairs=0, decay_mode="head", dt_softplus=True,
             two_endpoint=False, has_D=True)
    d.update(kw)
    return d


@pytest.mark.parametrize("kw,status", [
    (dict(), 0),
    (dict(nheads=3, ngroups=2), -2),            # groups must divide heads
    (dict(n_real=60), -2),                      # n_real + 2 n_pairs != dstate
    (dict(decay_mode="head", n_real=32, n_pairs=16), -2),  # pairs need per-row mode
    (dict(rank_in=2, rank_out=1), -2),          # D needs O == R
    (dict(rank_in=2, rank_out=1, has_D=False), 0),   # O != R without feedthrough
    (dict(rank_in=1, rank_out=4, has_D=False), 0),
    (dict(rank_in=8, rank_out=1, has_D=False), -5),  # widest rank the scans tile is 4
    (dict(headdim=24), -5),
    (dict(dstate=48, n_real=48), -5),
    (dict(decay_mode="coord", n_real=31, n_pairs=16, dstate=63), -5),
    (dict(seqlen=-1), -2),
    # static real rows: per-row mode only, at most n_real, an even count
    (dict(decay_mode="coord", n_real=32, n_pairs=16, n_static=8), 0),
    (dict(decay_mode="coord", n_real=32, n_pairs=16, n_static=32), 0),
    (dict(decay_mode="coord", n_real=32, n_pairs=16, n_static=34), -2),
    (dict(decay_mode="coord", n_real=32, n_pairs=16, n_static=-2), -2),
    (dict(decay_mode="coord", n_real=32, n_pairs=16, n_static=3), -5),
    (dict(n_static=2), -2),                     # head decay has no static rows
])
def test_descriptor_validation(kw, status):
    d = _lib.make_desc(base_desc(**kw), "bf16")
    assert ssm.check_desc(d) == status


def test_bad_dtype_and_flags():
    d = _lib.make_desc(base_desc(), "bf16")
    d.io_dtype = 7
    assert ssm.check_desc(d) == -3
    d = _lib.make_desc(base_desc(), "bf16")
    d.flags = 64
    assert ssm.check_desc(d) == -2


def test_chunk_and_saved_bytes():
    d = _lib.make_desc(base_desc(), "bf16")
    assert ssm.chunk_tokens(d) == 64
    nch = (100 + 63) // 64
    assert ssm.saved_bytes(d) == 2 * 4 * (nch + 1) * 64 * 64 * 2  # bf16 states
    df = _lib.make_desc(base_desc(dstate=32, n_real=32, headdim=16), "f32")  # fp32 states
    assert ssm.saved_bytes(df) == 2 * 4 * (nch + 1) * 32 * 16 * 4
    dh = _lib.make_desc(base_desc(decay_mode="coord", n_real=32, n_pairs=16, rank_in=2,
                                  rank_out=2, two_endpoint=True), "bf16")
    assert ssm.chunk_tokens(dh) == 16
    dh32 = _lib.make_desc(base_desc(decay_mode="coord", n_real=32, n_pairs=16, rank_in=2,
                                    rank_out=2, two_endpoint=True), "bf16", 32)
    assert ssm.chunk_tokens(dh32) == 32  # a chunk the caller asks for
    # the HybridMamba training step: the forward walks 32-token chunks, but the saved
    # states stay those of the 16-token plan chunks the reverse pass consumes
    dt = _lib.make_desc(dict(base_desc(decay_mode="coord", n_real=32, n_pairs=16, rank_in=2,
                                       rank_out=2, two_endpoint=True), batch=2, seqlen=16384,
                             nheads=32, ngroups=32), "bf16")
    assert ssm.chunk_tokens(dt) == 16
    assert ssm.saved_bytes(dt) == 2 * 32 * (16384 // 16 + 1) * 64 * 64 * 2


def test_null_pointers_rejected_before_launch():
    lib = ssm.load()
    d = _lib.make_desc(base_desc(), "bf16")
    args = _lib.SsmFwdArgs()
    assert lib.ssm_scan_fwd(ctypes.byref(d), ctypes.byref(args), None, 0, None) == -1
    assert lib.ssm_scan_fwd(ctypes.byref(d), None, None, 0, None) == -1
    assert lib.ssm_scan_fwd(None, ctypes.byref(args), None, 0, None) == -1
    # misaligned pointers (never dereferenced: validation fails first)
    fake = [0x1000 * (i + 1) for i in range(11)]
    args = _lib.SsmFwdArgs(*fake)
    args.omega = None
    args.beta = None
    args.gamma = None
    args.saved = None
    args.x = 0x1002
    assert lib.ssm_scan_fwd(ctypes.byref(d), ctypes.byref(args), None, 0, None) == -4
    # D given without the flag
    d2 = _lib.make_desc(base_desc(has_D=False), "bf16")
    args.x = 0x1000
    assert lib.ssm_scan_fwd(ctypes.byref(d2), ctypes.byref(args), None, 0, None) == -1


def header_struct_fields(name):
    """Member names of a typedef struct in include/ssm_scan.h, in declaration order."""
    import re
    text = open(os.path.join(ROOT, "include", "ssm_scan.h")).read()
    body = re.search(r"typedef struct \{([^{}]*)\}\s*" + name + ";", text).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    names = []
    for decl in body.split(";"):
        decl = decl.strip()
        if not decl:
            continue
        for part in decl.split(","):
            names.append(re.findall(r"[A-Za-z_][A-Za-z0-9_]*", part)[-1])
    return names


def test_ctypes_structs_match_header_layout():
    assert [f[0] for f in _lib.SsmDesc._fields_] == header_struct_fields("ssm_desc")
    assert [f[0] for f in _lib.SsmFwdArgs._fields_] == header_struct_fields("ssm_fwd_args")
    assert [f[0] for f in _lib.SsmBwdArgs._fields_] == header_struct_fields("ssm_bwd_args")
    assert [f[0] for f in _lib.SsmDecodeArgs._fields_] == header_struct_fields("ssm_decode_args")


def test_state_carry_pointers_must_be_aligned():
    lib = ssm.load()
    d = _lib.make_desc(base_desc(), "bf16")
    args = _lib.SsmFwdArgs(*[0x1000 * (i + 1) for i in range(11)])
    args.omega = args.beta = args.gamma = args.saved = None
    args.h0 = 0x2008  # 8-byte aligned only
    assert lib.ssm_scan_fwd(ctypes.byref(d), ctypes.byref(args), None, 0, None) == -4
    args.h0 = None
    args.h_final = 0x2004
    assert lib.ssm_scan_fwd(ctypes.byref(d), ctypes.byref(args), None, 0, None) == -4


def _decode_args(**kw):
    """Recurrent-step arguments with distinct fake (never dereferenced) pointers."""
    names = [f[0] for f in _lib.SsmDecodeArgs._fields_]
    a = _lib.SsmDecodeArgs(*[0x1000 * (i + 1) for i in range(len(names))])
    a.omega = a.beta = a.gamma = a.x_prev = a.B_prev = None
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("dkw,akw,status", [
    (dict(seqlen=2), {}, -2),                          # a step is one token
    (dict(rank_in=9, rank_out=9), {}, -5),             # rank above the step kernel's limit
    (dict(headdim=1028), {}, -5),
    (dict(dstate=512, n_real=512, rank_in=8, rank_out=8), {}, -5),  # tables exceed the LDS budget
    (dict(headdim=18), {}, -5),                        # 4 | headdim
    (dict(), dict(D=None), -1),                        # HAS_D without D
    (dict(), dict(x_prev=0x9000, B_prev=0x9100), -1),  # previous token without two-endpoint
    (dict(two_endpoint=True, decay_mode="coord", n_real=32, n_pairs=16, rank_in=2, rank_out=2),
     dict(omega=0x9000, beta=0x9100, gamma=0x9200, x_prev=0x9300), -1),  # x_prev without B_prev
    (dict(), dict(state=0x9004), -4),                  # state not 16-byte aligned
    (dict(), dict(state=None), -1),
])
def test_decode_step_validation_before_launch(dkw, akw, status):
    lib = ssm.load()
    d = _lib.make_desc(base_desc(**dict(dict(seqlen=1), **dkw)), "bf16")
    a = _decode_args(**akw)
    assert lib.ssm_decode_step(ctypes.byref(d), ctypes.byref(a), None) == status
    assert lib.ssm_decode_step(None, ctypes.byref(a), None) == -1
    assert lib.ssm_decode_step(ctypes.byref(d), None, None) in (-1, status)


# ---------------------------------------------------------------- binding argument checks
def _cpu_problem(name="hybrid", **kw):
    import torch

    import workloads
    spec = workloads.spec(name, batch=1, seqlen=20, nheads=2, ngroups=2, **kw)
    prob = workloads.make_problem(spec, seed=0, with_dy=True)
    io = torch.bfloat16 if prob["dtype"] == "bf16" else torch.float32
    t = {k: torch.from_numpy(prob[k]).to(io) for k in ("x", "B", "C", "dy")}
    for k in ("dt", "A", "omega", "beta", "gamma", "D"):
        if prob.get(k) is not None:
            t[k] = torch.from_numpy(prob[k]).contiguous()
    desc = _lib.make_desc(prob["desc"], prob["dtype"])
    t["y"] = torch.empty_like(t["dy"])
    return desc, t


def _fwd(desc, t, **over):
    a = dict(t)
    a.update(over)
    _lib.scan_fwd(desc, a["x"], a["B"], a["C"], a["dt"], a["A"], a["y"], omega=a.get("omega"),
                  beta=a.get("beta"), gamma=a.get("gamma"), D=a.get("D"))


@pytest.mark.parametrize("what", ["numel", "dtype", "layout", "device", "missing", "params"])
def test_binding_rejects_bad_tensors_before_the_call(what):
    """The ctypes wrappers check every tensor against the descriptor (element count,
    dtype, contiguity, GPU placement, required pointers) and raise before anything is
    enqueued: on this CPU-only host the checks are reached with host tensors."""
    import torch
    desc, t = _cpu_problem()
    if what == "numel":      # a tensor smaller than the descriptor implies
        bad, msg = dict(x=t["x"][:, :-1]), "elements"
    elif what == "dtype":    # fp32 where the io dtype is bf16
        bad, msg = dict(B=t["B"].float()), "expected"
    elif what == "layout":   # a strided view (e.g. a split of a packed projection)
        wide = torch.cat([t["C"], t["C"]], dim=-1)
        bad, msg = dict(C=wide[..., : t["C"].shape[-1]]), "contiguous"
    elif what == "device":   # every check passes but the tensors are on the host
        bad, msg = dict(), "GPU"
    elif what == "missing":  # two-endpoint writes need beta and gamma
        bad, msg = dict(beta=None), "required"
    else:                    # per-head rates of the wrong length
        bad, msg = dict(A=t["A"][:1]), "elements"
    with pytest.raises(_lib.SsmError, match=msg):
        _fwd(desc, t, **bad)


def test_binding_checks_gradient_and_step_tensors():
    import torch
    desc, t = _cpu_problem()
    saved = torch.empty(ssm.saved_bytes(desc) // 4 + 1, dtype=torch.float32)
    g = dict(dx=torch.empty_like(t["x"]), dB=torch.empty_like(t["B"]),
             dC=torch.empty_like(t["C"]), ddt=torch.empty_like(t["dt"]))
    with pytest.raises(_lib.SsmError, match="dB"):
        _lib.scan_bwd(desc, t["x"], t["B"], t["C"], t["dy"], t["dt"], t["A"], saved, g["dx"],
                      g["dB"][:, :-1], g["dC"], g["ddt"], omega=t["omega"], beta=t["beta"],
                      gamma=t["gamma"], D=t["D"])
    with pytest.raises(_lib.SsmError, match="saved"):
        _lib.scan_bwd(desc, t["x"], t["B"], t["C"], t["dy"], t["dt"], t["A"], saved[:8],
                      g["dx"], g["dB"], g["dC"], g["ddt"], omega=t["omega"], beta=t["beta"],
                      gamma=t["gamma"], D=t["D"])
    step = _lib.make_desc(dict(batch=1, seqlen=1, nheads=2, ngroups=2, headdim=64, dstate=64,
                               rank_in=2, rank_out=2, n_real=32, n_pairs=16, decay_mode="coord",
                               dt_softplus=True, two_endpoint=True, has_D=True), "bf16")
    x = t["x"][:, 0].contiguous()
    state = torch.empty(1, 2, 64, 64, dtype=torch.float32)
    with pytest.raises(_lib.SsmError, match="state"):
        _lib.decode_step(step, x, t["B"][:, 0].contiguous(), t["C"][:, 0].contiguous(),
                         t["dt"][:, 0].contiguous(), t["A"], state[:, :1], torch.empty_like(x),
                         omega=t["omega"], beta=t["beta"][:, 0].contiguous(),
                         gamma=t["gamma"][:, 0].contiguous(), D=t["D"])
