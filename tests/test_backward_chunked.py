"""The chunked backward algebra (tests/chunked_backward.py, which the HIP backward
kernels follow stage for stage) reproduces the oracle's gradients in fp64: ragged
and exact chunk counts, decay at the -5 floor and near zero, zero and nonzero
states and state cotangents."""
import numpy as np
import pytest

from oracle import backward_oracle
from tests.chunked_backward import chunked_backward


@pytest.mark.parametrize("T,g_lo,with_state", [(150, -5.0, True), (64, -0.05, True),
                                               (37, -5.0, False), (130, -1.0, True)])
def test_chunked_backward_matches_oracle(T, g_lo, with_state):
    rng = np.random.default_rng(T)
    H, dk, dv = 2, 8, 6
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = rng.uniform(g_lo, 0.0, (T, H, dk))
    beta = rng.uniform(0.0, 1.0, (T, H))
    s0 = rng.standard_normal((H, dk, dv)) * 0.3 if with_state else None
    d_out = rng.standard_normal((T, H, dv))
    d_fin = rng.standard_normal((H, dk, dv)) if with_state else None
    got = chunked_backward(q, k, v, g, beta, 0.5, d_out, s0, d_fin)
    ref = backward_oracle(q[None], k[None], v[None], g[None], beta[None], 0.5, d_out[None],
                          None if s0 is None else s0[None],
                          None if d_fin is None else d_fin[None])
    for name in ("dq", "dk", "dv", "dg", "dbeta", "ds0"):
        y = ref[name][0]
        err = np.linalg.norm(got[name] - y) / np.linalg.norm(y)
        assert err < 1e-12, f"{name}: {err:.3e}"
