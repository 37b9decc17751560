"""fp64 CPU oracle for the state-mediated selective SSM kernel.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU product
package never imports it; the two share no code (only the seeded input
generator in ``workloads.py`` serves both, and it holds none of the method's
arithmetic).

Contents
--------
* ``fwd`` / ``bwd``: ctypes front-end of ``ssm_oracle.c`` -- the plain
  sequential fp64 recurrence (and its hand-derived adjoint) of
  "When a Diagonal State Is Not Enough" (sungsoo.github.io), Part 01 and
  Part 03:  h_t = A_t h_{t-1} + gamma_t B_t X_t + beta_t B_{t-1} X_{t-1},
  y_t = C_t^T h_t + D X_t.
* ``forms``: small independent numpy/torch forms used to pin the recurrence
  (the O(L^2) masked-linear-attention form of Theorem 24, the complex-diagonal
  form of Theorem 8, the transfer operator C_t Phi_{t,s} B_s of Theorem 21).
"""
from .core import (  # noqa: F401
    OracleDesc,
    build,
    bwd,
    fwd,
    lib_path,
    load,
)
