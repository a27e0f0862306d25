"""CPU oracle for Kimi Delta Attention (KDA) -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  It shares no code with the
HIP path (``gated_delta_rule_102_amd``) and neither side imports the other;
the only thing both use is the seeded input generator module, which holds none
of the method's arithmetic.

Contents
  * ``kda_oracle.c`` -- the fp64 sequential recurrence in plain C (OpenMP over
    the independent (sequence, head) pairs), loaded through :mod:`ctypes`.
  * :func:`recurrence_np` -- the same definition written once more in numpy,
    used only to cross-check the C library on small shapes.
  * :func:`unrolled_np` -- the closed form obtained by unrolling the recurrence
    into products of the per-token transition matrices (brute force, T <= 8).
  * :func:`prologue_np` -- the gate/normalisation prologue (unit-norm q and k,
    g = max(-5, -softplus(x)), beta = sigmoid(x)) in fp64, for the fused path.
  * :func:`transition_np` -- a segment's transition (the product of the
    per-token maps with v = 0), for context parallelism, in fp64.
  * :func:`backward_oracle` -- gradients of the recurrence (dq, dk, dv, dg,
    dbeta, dS_0) by fp64 reverse-mode autodiff on the CPU (``grad.py``).

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, special cases and invariants; see the test docstrings.
"""
from .ref import (  # noqa: F401
    build,
    load,
    oracle_forward,
    prologue_np,
    recurrence_np,
    transition_np,
    unrolled_np,
    widen_np,
)
from .grad import backward_oracle  # noqa: F401
