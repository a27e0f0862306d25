"""Gradients of the KDA recurrence in fp64 -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use this module.  It shares nothing with the HIP path.

The forward rule is the per-token KDA recurrence (neurohive.io Kimi K3 review,
section "Sequence length: hybrid KDA and Gated MLA attention": a fixed-size
state per head that forgets per key channel and is written by a delta rule;
the log of the retention factor is bounded below at -5):

    S' = Diag(exp g_t) S,   delta_t = beta_t (v_t - S'^T k_t),
    S  = S' + k_t delta_t^T,   o_t = S^T (scale q_t).

The pages train the model at up to 1M tokens of context (best.xiaohu.ai
"Kimi K3 tech report", section on the context curriculum) but print no
backward pass, so the gradients are defined as the plain derivatives of that
rule: for a scalar loss

    L = sum_t <dO_t, o_t> + <dS_T, S_T>

(dO the cotangent of every output, dS_T that of the final state) the function
returns dL/dq, dL/dk, dL/dv, dL/dg, dL/dbeta and dL/dS_0.  They are obtained by
reverse-mode automatic differentiation (torch.autograd, a library primitive)
through the recurrence written with plain fp64 tensor operations on the CPU.

Parity status: pinned by ``tests/test_oracle_pins.py`` against central finite
differences of the C oracle's forward and against special cases whose
derivatives vanish exactly.
"""
from __future__ import annotations

import numpy as np
import torch

from .ref import widen_np


def _recurrence(q, k, v, g, beta, scale, s0):
    """The recurrence over T tokens for N independent (sequence, head) pairs.

    q, k, g: [N, T, dk]; v: [N, T, dv]; beta: [N, T]; s0: [N, dk, dv] (fp64 tensors).
    Returns (out [N, T, dv], S_T [N, dk, dv]).
    """
    S = s0
    outs = []
    for t in range(q.shape[1]):
        S = S * torch.exp(g[:, t])[:, :, None]                      # forget rows
        recall = (S * k[:, t, :, None]).sum(1)                      # S'^T k
        write = beta[:, t, None] * (v[:, t] - recall)               # beta (v - S'^T k)
        S = S + k[:, t, :, None] * write[:, None, :]                # + k delta^T
        outs.append((S * (scale * q[:, t, :, None])).sum(1))        # S^T (scale q)
    return torch.stack(outs, 1), S


def backward_oracle(q, k, v, g, beta, scale, d_out, initial_state=None, d_final=None):
    """Gradients of L = <d_out, out> + <d_final, final_state> for fixed-length inputs.

    Library layout: q, k, g [B, T, H, dk]; v, d_out [B, T, H, dv]; beta [B, T, H];
    initial_state, d_final [B, H, dk, dv] (None = zero).  Inputs may be bf16
    (torch tensors or uint16 bits), fp32 or fp64; they are widened exactly.
    Returns a dict of fp64 numpy arrays dq, dk, dv, dg, dbeta (input layouts) and
    ds0 [B, H, dk, dv].
    """
    q, k, v, g, beta, d_out = (widen_np(x) for x in (q, k, v, g, beta, d_out))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    s0 = np.zeros((B, H, dk, dv)) if initial_state is None else widen_np(initial_state)
    dsT = np.zeros((B, H, dk, dv)) if d_final is None else widen_np(d_final)

    def pairs(x):  # [B, T, H, ...] -> [B*H, T, ...]
        x = np.moveaxis(x, 2, 1)
        return torch.from_numpy(np.ascontiguousarray(x.reshape(B * H, T, *x.shape[3:])))

    leaves = [pairs(x).requires_grad_(True) for x in (q, k, v, g)]
    lb = pairs(beta).requires_grad_(True)
    ls0 = torch.from_numpy(s0.reshape(B * H, dk, dv).copy()).requires_grad_(True)
    with torch.enable_grad():
        out, sT = _recurrence(*leaves[:3], leaves[3], lb, float(scale), ls0)
        grads = torch.autograd.grad(
            (out, sT), (*leaves, lb, ls0),
            grad_outputs=(pairs(d_out), torch.from_numpy(dsT.reshape(B * H, dk, dv).copy())),
            allow_unused=False)

    def back(x):  # [B*H, T, ...] -> [B, T, H, ...]
        x = x.detach().numpy().reshape(B, H, T, *x.shape[2:])
        return np.ascontiguousarray(np.moveaxis(x, 1, 2))

    dq_, dk_, dv_, dg_, db_, ds0 = grads
    return dict(dq=back(dq_), dk=back(dk_), dv=back(dv_), dg=back(dg_), dbeta=back(db_),
                ds0=ds0.detach().numpy().reshape(B, H, dk, dv))
