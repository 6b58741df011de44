"""Float64 CPU oracle of the QSVD latent-attention path (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package.  The HIP library never imports or calls it.
"""
from .qsvd_oracle import *  # noqa: F401,F403
from . import qsvd_oracle as _m

__all__ = [n for n in dir(_m) if not n.startswith("_")]
