"""The chunked backward pass of KDA, in numpy fp64, stage by stage.

Test helper, not the oracle: it states the algebra the HIP backward kernels are
built on, stage for stage, so that a CPU test can show it agrees with the
oracle's gradients before (and independently of) the GPU code, and so that a
single GPU stage can be checked against its own intermediate.

Per (sequence, head) and chunk of C = 64 rows (a ragged last chunk is padded
with rows whose q, k, v, g, beta and output cotangent are zero), the forward is
written with the chunk's operands (G = running sum of g inside the chunk):

  A'[t,s] = sum_c k[t,c] k[s,c] e^{G[t,c]-G[s,c]}  (s < t),   Ti = (I + Diag(beta) A')^-1
  M'[t,s] = sum_c q[t,c] k[s,c] e^{G[t,c]-G[s,c]}  (s <= t),  Tb = Ti Diag(beta)
  Kg = k e^G,  W = Tb Kg,  P = scale M' Tb,  Q' = scale q e^G - P Kg,
  Kt = k e^{G_last - G},  Lam = e^{G_last}
  Delta = Tb V - W S,   O = Q' S + P V,   S_next = Lam S + Kt^T Delta

so one chunk is an affine map of (S, V).  The backward is then
  1. bwd_prep  : the operands above, per chunk (independent of the state);
  2. fwd scan  : S_c at every chunk start and Delta_c;
  3. bwd scan  : from dS = dS_T backwards, dU = Kt dS_next, dV = P^T dO + Tb^T dU,
                 dS_c = Lam dS_next + Q'^T dO - W^T dU;
  4. operand gradients (contractions over dv): dQ' = dO S^T, dW = -dU S^T,
     dKt = Delta dS_next^T, dLam = rowsum(S * dS_next), dP = dO V^T, dTb = dU V^T;
  5. the n x n algebra: dP_tot = dP - dQ' Kg^T, dKg = -P^T dQ' + Tb^T dW,
     dTb_tot = dTb + scale M'^T dP_tot + dW Kg^T, dM' = scale dP_tot Tb^T (s <= t),
     dbeta_s = sum_t Ti[t,s] dTb_tot[t,s] (column sums), dTi = dTb_tot Diag(beta),
     dA = -Ti^T dTi Ti^T (s < t), dbeta_t += sum_s dA[t,s] A'[t,s], dA' = Diag(beta) dA;
  6. the decayed products and the chain to q, k, g: with D = dA' or dM',
     X[t,c] = sum_s D[t,s] k[s,c] e^{G[t,c]-G[s,c]}  (row side)
     Z[s,c] = sum_t D[t,s] a[t,c] e^{G[t,c]-G[s,c]}  (column side, a = k or q)
     dq = scale dQ' e^G + X_M,
     dk = dKg e^G + dKt e^{G_last-G} + X_A + Z_A + Z_M,
     dG = q dq + k (dKg e^G + X_A - dKt e^{G_last-G} - Z_A - Z_M),
     plus sum_t dKt Kt + dLam Lam on the last row; dg = reverse running sum of dG.
The decayed products are formed with 16-row sub-tile references (the running
sum at the last row of each sub-tile) so that every factor stays inside fp32's
range while the log-decay is bounded below by -5 (neurohive.io Kimi K3 review,
section "Sequence length: hybrid KDA and Gated MLA attention").
"""
from __future__ import annotations

import numpy as np

C, BLK = 64, 16


def _refs(G):
    nb = G.shape[0] // BLK
    R = np.stack([G[(b + 1) * BLK - 1] for b in range(nb)])          # [nb, dk]
    blk = np.arange(G.shape[0]) // BLK
    return R, blk, np.exp(G - R[blk]), np.exp(R[blk] - G)            # rowf >= 1, colf <= 1


def _pair_gram(a_row, b_col, R, lower_incl):
    """sum_c a_row[t,c] f_IJ[c] b_col[s,c] per sub-tile pair (J <= I), masked."""
    n = a_row.shape[0]
    out = np.zeros((n, n))
    for I in range(n // BLK):
        for J in range(I + 1):
            f = np.exp(R[I] - R[J]) if J < I else np.ones(R.shape[1])
            ti, sj = slice(I * BLK, (I + 1) * BLK), slice(J * BLK, (J + 1) * BLK)
            out[ti, sj] = (a_row[ti] * f) @ b_col[sj].T
    mask = np.tril(np.ones((n, n)), 0 if lower_incl else -1)
    return out * mask


def bwd_prep(q, k, g, beta, scale):
    """Stage 1 on one padded chunk (q, k, g [C, dk]; beta [C])."""
    G = np.cumsum(g, axis=0)
    R, blk, rowf, colf = _refs(G)
    Ap = _pair_gram(k * rowf, k * colf, R, False)
    Mp = _pair_gram(q * rowf, k * colf, R, True)
    Ti = np.linalg.inv(np.eye(C) + beta[:, None] * Ap)
    Tb = Ti * beta[None, :]
    Kg = k * np.exp(G)
    W = Tb @ Kg
    P = scale * Mp @ Tb
    Qp = scale * q * np.exp(G) - P @ Kg
    Kt = k * np.exp(G[-1] - G)
    return dict(G=G, Ap=Ap, Mp=Mp, Ti=Ti, Tb=Tb, W=W, P=P, Qp=Qp, Kt=Kt, Lam=np.exp(G[-1]))


def _decayed(D, c_row, c_col, G):
    """(X, Z): X[t] = sum_s D[t,s] c_col[s] e^{G_t-G_s}, Z[s] = sum_t D[t,s] c_row[t] e^{G_t-G_s}."""
    R, blk, rowf, colf = _refs(G)
    X = np.zeros_like(c_col)
    Z = np.zeros_like(c_row)
    for I in range(C // BLK):
        for J in range(I + 1):
            f = np.exp(R[I] - R[J]) if J < I else np.ones(G.shape[1])
            ti, sj = slice(I * BLK, (I + 1) * BLK), slice(J * BLK, (J + 1) * BLK)
            X[ti] += f * (D[ti, sj] @ (c_col[sj] * colf[sj]))
            Z[sj] += f * (D[ti, sj].T @ (c_row[ti] * rowf[ti]))
    return X * rowf, Z * colf


def chunked_backward(q, k, v, g, beta, scale, d_out, initial_state=None, d_final=None):
    """Gradients for one sequence, all heads.  q,k,g [T,H,dk]; v,d_out [T,H,dv];
    beta [T,H]; states [H,dk,dv].  Returns dq, dk, dv, dg, dbeta, ds0 (fp64)."""
    T, H, dk = q.shape
    dv = v.shape[-1]
    nc = -(-T // C)
    pad = nc * C - T

    def padded(x):
        return np.concatenate([x, np.zeros((pad, *x.shape[1:]))]) if pad else x

    q, k, v, g, beta, d_out = (padded(np.asarray(x, float)) for x in (q, k, v, g, beta, d_out))
    res = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dg", g),
                                            ("dbeta", beta))}
    ds0 = np.zeros((H, dk, dv))
    for h in range(H):
        ch = [slice(c * C, (c + 1) * C) for c in range(nc)]
        ops = [bwd_prep(q[s, h], k[s, h], g[s, h], beta[s, h], scale) for s in ch]
        S = np.zeros((dk, dv)) if initial_state is None else np.array(initial_state[h], float)
        Ss, Dl = [], []
        for c, s in enumerate(ch):                                   # stage 2
            o = ops[c]
            Ss.append(S)
            Dl.append(o["Tb"] @ v[s, h] - o["W"] @ S)
            S = o["Lam"][:, None] * S + o["Kt"].T @ Dl[-1]
        dS = np.zeros((dk, dv)) if d_final is None else np.array(d_final[h], float)
        dSn, dU = [None] * nc, [None] * nc
        for c in reversed(range(nc)):                                # stage 3
            o, s = ops[c], ch[c]
            dSn[c] = dS
            dU[c] = o["Kt"] @ dS
            res["dv"][s, h] = o["P"].T @ d_out[s, h] + o["Tb"].T @ dU[c]
            dS = o["Lam"][:, None] * dS + o["Qp"].T @ d_out[s, h] - o["W"].T @ dU[c]
        ds0[h] = dS
        for c, s in enumerate(ch):                                   # stages 4-6
            o = ops[c]
            dO, V = d_out[s, h], v[s, h]
            dQp = dO @ Ss[c].T
            dW = -dU[c] @ Ss[c].T
            dKt = Dl[c] @ dSn[c].T
            dLam = (Ss[c] * dSn[c]).sum(1)
            dP = dO @ V.T
            dTb = dU[c] @ V.T
            G = o["G"]
            Kg = k[s, h] * np.exp(G)
            dPt = dP - dQp @ Kg.T
            dKg = -o["P"].T @ dQp + o["Tb"].T @ dW
            dTbt = dTb + scale * o["Mp"].T @ dPt + dW @ Kg.T
            dMp = scale * np.tril(dPt @ o["Tb"].T)
            db = (o["Ti"] * dTbt).sum(0)
            dTi = dTbt * beta[s, h][None, :]
            dA = -np.tril(o["Ti"].T @ dTi @ o["Ti"].T, -1)
            db += (dA * o["Ap"]).sum(1)
            dAp = beta[s, h][:, None] * dA
            XA, ZA = _decayed(dAp, k[s, h], k[s, h], G)
            XM, ZM = _decayed(dMp, q[s, h], k[s, h], G)
            e, et = np.exp(G), np.exp(G[-1] - G)
            dq = scale * dQp * e + XM
            dkk = dKg * e + dKt * et + XA + ZA + ZM
            dG = q[s, h] * dq + k[s, h] * (dKg * e + XA - dKt * et - ZA - ZM)
            dG[-1] += (dKt * k[s, h] * et).sum(0) + dLam * o["Lam"]
            res["dq"][s, h], res["dk"][s, h] = dq, dkk
            res["dg"][s, h] = np.cumsum(dG[::-1], axis=0)[::-1]
            res["dbeta"][s, h] = db
    return {n: x[:T] for n, x in res.items()} | {"ds0": ds0}
