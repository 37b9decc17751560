"""MI355X-native state-mediated selective SSM scan and recurrent step (SISO, SSD-MIMO,
HybridMamba rows).

The computation lives in hand-written HIP kernels for gfx950 behind the C ABI of
``include/ssm_scan.h`` (``libssmscan.so``); this package is the thin ctypes
binding plus a torch-facing wrapper that allocates outputs and workspaces.
"""
from ._lib import (  # noqa: F401
    EXPORTS,
    SSM_BF16,
    SSM_DECAY_COORD,
    SSM_DECAY_HEAD,
    SSM_F32,
    SSM_F_DT_SOFTPLUS,
    SSM_F_HAS_D,
    SSM_F_TWO_ENDPOINT,
    SsmDesc,
    SsmError,
    check_desc,
    chunk_tokens,
    load,
    make_desc,
    saved_bytes,
    scan_bwd,
    scan_fwd,
    scan_fwd_noalloc,
    scratch_bytes,
    workspace_bytes,
)
from .scan import backward, decode_step, forward  # noqa: F401
