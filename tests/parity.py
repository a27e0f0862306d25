"""Comparison helpers shared by the GPU parity tests (tolerances, oracle calls).

Tolerances (written here once, used by every GPU test):
  bf16 inputs: max-abs <= 2e-2 AND rel-L2 <= 1e-2, on outputs and final states;
  fp32 inputs: rel-L2 <= 1e-4.
rel-L2 is ||x - y||_2 / ||y||_2 over the whole compared tensor.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from oracle import oracle_forward

TOL = {torch.bfloat16: dict(max_abs=2e-2, rel_l2=1e-2), torch.float32: dict(max_abs=None, rel_l2=1e-4)}


def errors(x, y):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    diff = x - y
    ref = np.linalg.norm(y)
    rel = np.linalg.norm(diff) / (ref if ref > 0 else 1.0)
    return float(np.max(np.abs(diff))) if diff.size else 0.0, float(rel)


def assert_close(name, got, ref, dtype):
    tol = TOL[dtype]
    got = got.detach().float().cpu().numpy() if isinstance(got, torch.Tensor) else got
    max_abs, rel = errors(got, ref)
    msg = f"{name}: max_abs={max_abs:.3e} rel_l2={rel:.3e} (tol {tol})"
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert rel <= tol["rel_l2"], msg
    if tol["max_abs"] is not None:
        assert max_abs <= tol["max_abs"], msg
    return max_abs, rel


def oracle_fixed(d, pairs=None, nthreads=0):
    """Oracle for fixed-length inputs d (tensors [B,T,H,.] on any device)."""
    cpu = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    B, T = cpu["q"].shape[:2]
    return oracle_forward(cpu["q"], cpu["k"], cpu["v"], cpu["g"], cpu["beta"], d["scale"],
                          B=B, T=T, initial_state=cpu.get("initial_state"), pairs=pairs,
                          nthreads=nthreads)


def oracle_pair_slices(d, pairs, bounds, workers=8):
    """Oracle on selected (sequence, head) pairs, extracting each pair's slice first.

    bounds[n] = (token_start, length) in the packed layout; tensors are [.., tokens, H, .].
    Returns a list of (out [len, dv], final [dk, dv]) in pair order.
    """
    H = d["q"].shape[-2]

    def flat(t):
        return t.reshape(-1, *t.shape[-2:]) if t.dim() > 2 else t.reshape(-1, t.shape[-1])

    q, k, v, g = (flat(d[x]) for x in ("q", "k", "v", "g"))
    beta = d["beta"].reshape(-1, H)
    s0 = d.get("initial_state")

    def one(pair):
        n, h = pair
        a, L = bounds[n]
        sl = slice(a, a + L)
        args = [x[sl, h:h + 1].cpu() for x in (q, k, v, g)]
        b = beta[sl, h:h + 1].cpu()
        init = None if s0 is None else s0[n, h:h + 1].unsqueeze(0).cpu()
        out, sT = oracle_forward(*args, b, d["scale"], B=1, T=L, initial_state=init, nthreads=1)
        return out[:, 0], sT[0]

    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(one, pairs))


class ErrAccum:
    """Max-abs and rel-L2 over a tensor compared piece by piece.

    rel-L2 = sqrt(sum (x - y)^2) / sqrt(sum y^2) over every piece added, so a whole
    full-size tensor is held to the same bar as in ``assert_close`` without ever
    holding all of it in fp64 at once."""

    def __init__(self, name, dtype):
        self.name, self.dtype = name, dtype
        self.sq_diff = 0.0
        self.sq_ref = 0.0
        self.max_abs = 0.0
        self.count = 0

    def add(self, got, ref):
        got = got.detach().float().cpu().numpy() if isinstance(got, torch.Tensor) else got
        x = np.asarray(got, dtype=np.float64)
        y = np.asarray(ref, dtype=np.float64)
        if x.shape != y.shape:
            raise ValueError(f"{self.name}: shapes {x.shape} and {y.shape} differ")
        assert np.all(np.isfinite(x)), f"{self.name}: non-finite values"
        diff = x - y
        self.sq_diff += float(np.dot(diff.ravel(), diff.ravel()))
        self.sq_ref += float(np.dot(y.ravel(), y.ravel()))
        if diff.size:
            self.max_abs = max(self.max_abs, float(np.max(np.abs(diff))))
        self.count += x.size

    def rel_l2(self):
        return (self.sq_diff ** 0.5) / (self.sq_ref ** 0.5 if self.sq_ref > 0 else 1.0)

    def check(self):
        tol = TOL[self.dtype]
        rel = self.rel_l2()
        msg = (f"{self.name}: max_abs={self.max_abs:.3e} rel_l2={rel:.3e} over "
               f"{self.count} values (tol {tol})")
        print(msg, flush=True)
        assert self.count > 0, f"{self.name}: nothing compared"
        assert rel <= tol["rel_l2"], msg
        if tol["max_abs"] is not None:
            assert self.max_abs <= tol["max_abs"], msg
        return self.max_abs, rel
