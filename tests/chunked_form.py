"""The chunked (blocked-over-time) form of KDA, in numpy fp64.

Test helper, not the oracle: it states the algebra the HIP prefill kernel is
built on, so that the tests can show that algebra agrees with the sequential
recurrence (the oracle) before any kernel exists, and can expose the per-chunk
intermediates when a kernel stage has to be checked on its own.

Per (sequence, head), for a chunk of n <= C tokens entering with state S
(dk x dv, rows are key channels), with G = cumsum of g over the chunk's tokens
(n x dk):

  A[t, s]  = beta_t * sum_c k[t,c] k[s,c] exp(G[t,c] - G[s,c])     (s < t, else 0)
  M[t, s]  = scale  * sum_c q[t,c] k[s,c] exp(G[t,c] - G[s,c])     (s <= t, else 0)
  Tinv     = (I + A)^-1                                           (unit lower triangular)
  Kbar     = k * exp(G),   Qbar = scale * q * exp(G),   Ktil = k * exp(G[n-1] - G)
  X        = V - Kbar S                       (what the decayed memory fails to recall)
  Delta    = Tinv Diag(beta) X                (the per-token writes, all at once)
  O        = Qbar S + M Delta
  S_next   = Diag(exp G[n-1]) S + Ktil^T Delta

Derivation: unrolling S_t = D_t S_{t-1} + k_t d_t^T inside the chunk gives
S_t = Diag(e^{G_t}) S + sum_{s<=t} Diag(e^{G_t - G_s}) k_s d_s^T; substituting into
d_t = beta_t (v_t - (D_t S_{t-1})^T k_t) gives (I + A) Delta = Diag(beta) X.

`subtile_factors` shows the overflow-safe split used on the GPU: with the
log-decay bounded below by -5 (neurohive.io Kimi K3 review, section "Sequence
length: hybrid KDA and Gated MLA attention"), referencing each 16-row sub-tile to
the cumulative decay at the end of that sub-tile keeps every factor within
[e^-80, e^80], inside the range of bf16 and fp32.
"""
from __future__ import annotations

import numpy as np


def chunk_step(q, k, v, g, beta, S, scale):
    """One chunk. q,k,g: [n,dk]; v: [n,dv]; beta: [n]; S: [dk,dv] -> (O, S_next, parts)."""
    n = q.shape[0]
    G = np.cumsum(g, axis=0)
    diff = G[:, None, :] - G[None, :, :]                      # [t, s, c]
    with np.errstate(over="ignore"):
        E = np.exp(np.where(np.arange(n)[:, None, None] >= np.arange(n)[None, :, None],
                            diff, -np.inf))                   # masked above the diagonal
    A = beta[:, None] * np.einsum("tc,sc,tsc->ts", k, k, E)
    A = np.tril(A, -1)
    M = scale * np.tril(np.einsum("tc,sc,tsc->ts", q, k, E))
    Tinv = np.linalg.inv(np.eye(n) + A)
    Kbar = k * np.exp(G)
    Qbar = scale * q * np.exp(G)
    Ktil = k * np.exp(G[-1][None, :] - G)
    X = v - Kbar @ S
    Delta = Tinv @ (beta[:, None] * X)
    O = Qbar @ S + M @ Delta
    S_next = np.exp(G[-1])[:, None] * S + Ktil.T @ Delta
    return O, S_next, dict(A=A, M=M, Tinv=Tinv, X=X, Delta=Delta, G=G)


def chunked_forward(q, k, v, g, beta, scale, C=64, initial_state=None):
    """Whole sequence, one head at a time. q,k,g: [T,H,dk]; v: [T,H,dv]; beta: [T,H]."""
    T, H, dk = q.shape
    dv = v.shape[-1]
    out = np.zeros((T, H, dv))
    final = np.zeros((H, dk, dv))
    for h in range(H):
        S = np.zeros((dk, dv)) if initial_state is None else np.array(initial_state[h], float)
        for c0 in range(0, T, C):
            sl = slice(c0, min(T, c0 + C))
            O, S, _ = chunk_step(q[sl, h], k[sl, h], v[sl, h], g[sl, h], beta[sl, h], S, scale)
            out[sl, h] = O
        final[h] = S
    return out, final


def subtile_factors(g, block=16):
    """Sub-tile decay factors of one chunk, referenced to each sub-tile's end.

    g: [n, dk] log-decays.  Returns a dict of the factors and the Gram it yields:
      rowf[t] = exp(G_t - R_b)  in [1, e^{5*block}]   (row side, b = sub-tile of t)
      colf[s] = exp(R_b - G_s)  in [e^{-5*block}, 1]  (column side, b = sub-tile of s)
      pair[(I, J)] = exp(R_I - R_J) <= 1 for J < I  (carries a column sub-tile J to row
      sub-tile I's reference), where R_b is G at the last row of sub-tile b.
    so that exp(G_t - G_s) = rowf[t] * pair[(I, J)] * colf[s] for s in J, t in I.
    """
    n, dk = g.shape
    G = np.cumsum(g, axis=0)
    nb = (n + block - 1) // block
    R = np.stack([G[min(n, (b + 1) * block) - 1] for b in range(nb)])   # [nb, dk]
    blk = np.arange(n) // block
    rowf = np.exp(G - R[blk])
    colf = np.exp(R[blk] - G)
    pair = {(I, J): np.exp(R[I] - R[J]) for I in range(nb) for J in range(I)}
    return dict(G=G, R=R, rowf=rowf, colf=colf, pair=pair, blk=blk)


def gram_from_subtiles(a, b, g, block=16):
    """sum_c a[t,c] b[s,c] exp(G_t - G_s) for s <= t, via the bounded sub-tile factors."""
    f = subtile_factors(g, block)
    n = a.shape[0]
    out = np.zeros((n, n))
    for t in range(n):
        for s in range(t + 1):
            I, J = f["blk"][t], f["blk"][s]
            col = b[s] * f["colf"][s] * (f["pair"][(I, J)] if J < I else 1.0)
            out[t, s] = np.sum(a[t] * f["rowf"][t] * col)
    return out
