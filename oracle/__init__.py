"""CPU oracle for the delta-rule recurrence (fp64, token by token).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the GPU library.
"""

from .backward import backward
from .preconditioner import precond_scan, surrogate, surrogate_grad
from .recurrence import forward, gate_kind, recurrent_step, rel_l2

__all__ = ["backward", "forward", "gate_kind", "precond_scan", "recurrent_step", "rel_l2", "surrogate", "surrogate_grad"]
