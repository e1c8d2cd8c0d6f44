"""fp64 CPU oracle of the GDLA forward pass.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the benchmark's
CPU-baseline leg, never by the GPU library or its Python binding.  It shares no code with the GPU
path.  Every function is pinned by the CPU tests (worked example, closed forms, invariants, library
routines, high-precision brute force); the RoPE convention is a reading, pinned only in its
mechanics (relative-position invariance, norm preservation), not in its frequencies or pairing.
"""

from .gdla_ref import *  # noqa: F401,F403
from .gdla_ref import __all__ as _ref_all
from .mla_ref import mla_forward

__all__ = list(_ref_all) + ["mla_forward"]
