"""Loader for the C oracle plus two small numpy formulations used to check it.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Nothing here may be
imported by the product path.

Shapes follow the library's layout: q, k, g are ``[total_T, H, dk]``, v is
``[total_T, H, dv]``, beta is ``[total_T, H]``, states are ``[N, H, dk, dv]``
with rows indexed by key channel.  Sequences are described either by
``(B, T)`` (B sequences of length T laid out back to back) or by
``cu_seqlens`` (N+1 monotone token offsets).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None

_BF16, _F32, _F64 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile ``kda_oracle.c`` with gcc -O2 (no fast-math) and OpenMP."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def load():
    """Load (building first if needed) the C oracle library."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        vp, i32, i64p, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_double
        lib.orc_kda_forward.argtypes = [vp, vp, vp, vp, vp, i32, vp, i32, i64p, i64p,
                                        i32, i32, i32, i32, dbl, vp, i32, vp, i32, vp, i32]
        lib.orc_kda_forward.restype = i32
        lib.orc_abi_version.restype = i32
        _lib = lib
    return _lib


def _as_np(x):
    """numpy view of an array or CPU torch tensor; bf16 becomes its uint16 bits."""
    if x is None:
        return None, None
    if type(x).__module__.startswith("torch"):
        if str(x.dtype) == "torch.bfloat16":
            import torch  # only reached when the caller already uses torch
            a = x.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
            return a, _BF16
        x = x.detach().contiguous().cpu().numpy()
    a = np.ascontiguousarray(x)
    if a.dtype == np.uint16:
        return a, _BF16
    if a.dtype == np.float32:
        return a, _F32
    if a.dtype == np.float64:
        return a, _F64
    raise TypeError(f"unsupported oracle input dtype {a.dtype}")


def widen_np(x) -> np.ndarray:
    """Exact widening of a bf16 (uint16 bits) / fp32 / fp64 array to float64."""
    a, code = _as_np(x)
    if code == _BF16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _seq_bounds(B, T, cu_seqlens):
    if cu_seqlens is not None:
        cu = np.asarray(cu_seqlens, dtype=np.int64).reshape(-1)
        return cu[:-1].copy(), np.diff(cu).astype(np.int64)
    start = np.arange(B, dtype=np.int64) * T
    return start, np.full(B, T, dtype=np.int64)


def oracle_forward(q, k, v, g, beta, scale, *, B=None, T=None, cu_seqlens=None,
                   initial_state=None, pairs=None, store_out=True, packed=False,
                   nthreads=0):
    """Run the fp64 C oracle.

    Inputs may be numpy arrays or CPU torch tensors (bf16, fp32 or fp64); q, k,
    v, g and beta must share one precision.  ``q``... may carry a leading batch
    axis (``[B, T, H, d]``) or be packed (``[total_T, H, d]``).

    Returns ``(out, final_state)`` as float64 arrays.  ``out`` is
    ``[total_T, H, dv]`` (rows of pairs that were not computed stay zero), or,
    with ``packed=True``, a list with one ``[len_n, dv]`` array per pair;
    ``final_state`` is ``[npairs, dk, dv]`` in pair order (all pairs in (n, h)
    order when ``pairs`` is None).
    """
    arrs = [_as_np(x) for x in (q, k, v, g, beta)]
    codes = {c for _, c in arrs}
    if len(codes) != 1:
        raise TypeError("q, k, v, g, beta must share one precision")
    in_code = codes.pop()
    qa, ka, va, ga, ba = [a for a, _ in arrs]
    H, dk = qa.shape[-2], qa.shape[-1]
    dv = va.shape[-1]
    total_T = qa.size // (H * dk)
    if B is None and cu_seqlens is None:
        if qa.ndim != 4:
            raise ValueError("give B and T, cu_seqlens, or [B, T, H, d] inputs")
        B, T = qa.shape[0], qa.shape[1]
    start, length = _seq_bounds(B, T, cu_seqlens)
    N = len(start)
    if int(start[-1] + length[-1]) > total_T:
        raise ValueError("sequences run past the end of the inputs")
    s0, s0_code = _as_np(initial_state)
    if pairs is None:
        pair_arr = None
        P = N * H
        pair_list = [(n, h) for n in range(N) for h in range(H)]
    else:
        pair_list = [(int(n), int(h)) for n, h in pairs]
        pair_arr = np.asarray(pair_list, dtype=np.int32).reshape(-1, 2)
        P = len(pair_list)
    if packed:
        out = np.zeros(int(sum(length[n] for n, _ in pair_list)) * dv, dtype=np.float64)
    else:
        out = np.zeros((total_T, H, dv), dtype=np.float64) if store_out else None
    sT = np.zeros((P, dk, dv), dtype=np.float64)
    lib = load()

    def ptr(a):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    rc = lib.orc_kda_forward(ptr(qa), ptr(ka), ptr(va), ptr(ga), ptr(ba), in_code,
                             ptr(s0), 0 if s0 is None else s0_code,
                             ptr(start), ptr(length), N, H, dk, dv, float(scale),
                             ptr(pair_arr), P, ptr(out) if (store_out or packed) else None,
                             1 if packed else 0, ptr(sT), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle returned {rc}")
    if packed:
        pieces, off = [], 0
        for n, _ in pair_list:
            L = int(length[n])
            pieces.append(out[off:off + L * dv].reshape(L, dv))
            off += L * dv
        return pieces, sT
    return out, sT


def recurrence_np(q, k, v, g, beta, scale, initial_state=None):
    """The recurrence once more, in numpy fp64, for one sequence.

    q, k, g: [T, H, dk]; v: [T, H, dv]; beta: [T, H]; initial_state [H, dk, dv].
    Returns (out [T, H, dv], final_state [H, dk, dv]).  Used only to
    cross-check the C library; small shapes only.
    """
    q, k, v, g, beta = (widen_np(x) for x in (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((H, dk, dv)) if initial_state is None else widen_np(initial_state).copy()
    out = np.zeros((T, H, dv))
    for t in range(T):
        S = S * np.exp(g[t])[:, :, None]                       # forget rows
        recall = np.einsum("hij,hi->hj", S, k[t])              # S^T k
        write = beta[t][:, None] * (v[t] - recall)             # beta (v - S^T k)
        S = S + k[t][:, :, None] * write[:, None, :]           # k write^T
        out[t] = np.einsum("hij,hi->hj", S, scale * q[t])      # S^T (scale q)
    return out, S


def unrolled_np(q, k, v, g, beta, scale, initial_state=None):
    """Brute force: unroll the recurrence into transition-matrix products.

    With M_t = (I - beta_t k_t k_t^T) Diag(exp g_t) and Phi(t, s) = M_t ... M_{s+1}
    (Phi(t, t) = I), the state after token t is
        S_t = Phi(t, -1) S_0 + sum_{s <= t} Phi(t, s) beta_s k_s v_s^T
    and o_t = S_t^T (scale q_t).  Every Phi is formed as an explicit dense
    product, so this is O(T^2 d^3): tiny shapes only (T <= 8, d <= 8).
    """
    q, k, v, g, beta = (widen_np(x) for x in (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[-1]
    S0 = np.zeros((H, dk, dv)) if initial_state is None else widen_np(initial_state)
    out = np.zeros((T, H, dv))
    final = np.zeros((H, dk, dv))
    eye = np.eye(dk)
    for h in range(H):
        Ms = [(eye - beta[t, h] * np.outer(k[t, h], k[t, h])) @ np.diag(np.exp(g[t, h]))
              for t in range(T)]

        def phi(t, s):
            P = eye.copy()
            for u in range(s + 1, t + 1):
                P = Ms[u] @ P
            return P

        for t in range(T):
            St = phi(t, -1) @ S0[h]
            for s in range(t + 1):
                St = St + phi(t, s) @ (beta[s, h] * np.outer(k[s, h], v[s, h]))
            out[t, h] = St.T @ (scale * q[t, h])
            if t == T - 1:
                final[h] = St
    return out, final


def transition_np(k, g, beta):
    """Transition of one segment, in fp64, from its definition: with v = 0 a token
    maps the state by M_t = (I - beta_t k_t k_t^T) Diag(exp g_t) (the recurrence of
    the C oracle with its write term removed), so the segment's exit state from an
    entry state S is P S with P = M_{T-1} ... M_1 M_0.  k, g: [T, H, dk];
    beta: [T, H].  Returns P [H, dk, dk].  Used for context parallelism, where a
    segment's exit state is P S_entry plus its zero-entry exit state."""
    k, g, beta = (widen_np(x) for x in (k, g, beta))
    T, H, dk = k.shape
    P = np.broadcast_to(np.eye(dk), (H, dk, dk)).copy()
    for t in range(T):
        P = P * np.exp(g[t])[:, :, None]                                  # Diag(e^g) P
        P = P - beta[t][:, None, None] * k[t][:, :, None] * np.einsum("hi,hij->hj", k[t], P)[:, None, :]
    return P


def prologue_np(q_raw, k_raw, g_raw, beta_raw, eps=1e-6, floor=-5.0):
    """The gate/normalisation prologue, in fp64, written out from its definitions.

    The pages bound the log of KDA's per-channel retention factor below at -5
    (neurohive.io Kimi K3 review, "Sequence length: hybrid KDA and Gated MLA
    attention") but print no gate formula; the reading used is
        q = q_raw / sqrt(sum_c q_raw^2 + eps),  k likewise (per token and head),
        g = max(floor, -softplus(g_raw)),  softplus(x) = log(1 + e^x),
        beta = sigmoid(beta_raw) = 1 / (1 + e^-x).
    Inputs are widened exactly (bf16 bits or fp32) to fp64; returns fp64 arrays.
    """
    q, k, g, b = (widen_np(x) for x in (q_raw, k_raw, g_raw, beta_raw))
    qn = q / np.sqrt((q * q).sum(-1, keepdims=True) + eps)
    kn = k / np.sqrt((k * k).sum(-1, keepdims=True) + eps)
    gg = np.maximum(floor, -np.logaddexp(0.0, g))      # log(1 + e^x) without overflow
    bb = 0.5 * (1.0 + np.tanh(0.5 * b))                # = 1 / (1 + e^-x), no overflow
    return qn, kn, gg, bb
