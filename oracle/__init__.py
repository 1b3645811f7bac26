"""fp64 CPU oracle for the gated delta-rule recurrence.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path. It shares no code with
the HIP kernels.

* ``recurrence`` -- the token-by-token recurrence in plain C (``kda_oracle.c``),
  fp64, OpenMP over independent (sequence, head) pairs, its reverse-mode
  gradient (``bwd``), and the variant with decoupled erase and write gates
  (``fwd_ew``, ``decode_step_ew``).
* ``dense`` -- a second, independent formulation for tiny inputs: explicit
  dense transition matrices and their products.
* ``gauge`` -- the gauge transform of Complex KDA onto positive gates
  (cumulative gate signs folded into q and k), in numpy.
"""
from .recurrence import build, bwd, bwd_ew, fwd, decode_step, decode_step_ew, fwd_ew, fwd_heads, threads  # noqa: F401
