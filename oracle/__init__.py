"""fp64 CPU oracle for the Mesa layer (test infrastructure only).

Imported only by ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py``.  It shares no code with the HIP path.
"""
from .mesa_oracle import cg_solve, cholesky_solve, mesa_forward, mesa_decode_step, diag_or_full, qk_preprocess, mesa_backward  # noqa: F401
