"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

The pages describe KDA in words only (no printed equation, no worked numbers):
a fixed-size state per head updated by a delta rule that forgets and writes,
with a per-key-channel retention factor whose log is bounded below at -5
(neurohive.io Kimi K3 review, section "Sequence length: hybrid KDA and Gated
MLA attention"; best.xiaohu.ai "Kimi K3 tech report", section "Sequence length:
replacing most attention layers with fixed-size memory").  So the oracle is
pinned by facts that hold for that reading independently of how the oracle is
coded: a hand-worked example, closed forms of special cases, brute force
unrolling, algebraic invariants, and the chunked algebra the GPU kernel uses.
A final test plants plausible mistakes in a copy of the recurrence and shows the
pins catch each one.
"""
import os

import numpy as np
import pytest

import oracle
from oracle import oracle_forward, recurrence_np, unrolled_np
from tests import chunked_form as cf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng_global = np.random.default_rng(1234)


def _rand_inputs(T, H, dk, dv, rng, g_lo=-5.0, g_hi=0.0, beta_lo=0.0, beta_hi=1.0,
                 unit=True):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = rng.uniform(g_lo, g_hi, (T, H, dk))
    beta = rng.uniform(beta_lo, beta_hi, (T, H))
    return q, k, v, g, beta


def run(q, k, v, g, beta, scale=1.0, s0=None):
    """Oracle on one sequence given as [T,H,*] arrays; returns out [T,H,dv], S [H,dk,dv]."""
    T = q.shape[0]
    init = None if s0 is None else s0[None]
    out, sT = oracle_forward(q, k, v, g, beta, scale, B=1, T=T, initial_state=init)
    return out, sT


# ---------------------------------------------------------------- hand-worked


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                key, *nums = line.split()
                vals[key] = np.array([float(x) for x in nums])
    return vals


def test_handworked_example():
    """A two-token, 2x2 example worked out by hand (tests/golden/handworked_2x2.txt)."""
    d = _read_golden("handworked_2x2.txt")
    q = np.stack([d["q1"], d["q2"]])[:, None, :]
    k = np.stack([d["k1"], d["k2"]])[:, None, :]
    v = np.stack([d["v1"], d["v2"]])[:, None, :]
    g = np.stack([d["g1"], d["g2"]])[:, None, :]
    beta = np.array([d["beta1"][0], d["beta2"][0]])[:, None]
    s0 = d["S0"].reshape(1, 2, 2)
    out, sT = run(q, k, v, g, beta, 1.0, s0)
    np.testing.assert_allclose(out[0, 0], d["o1"], atol=1e-12)
    np.testing.assert_allclose(out[1, 0], d["o2"], atol=1e-12)
    np.testing.assert_allclose(sT[0].reshape(-1), d["S2"], atol=1e-12)


# ---------------------------------------------------------------- brute force


@pytest.mark.parametrize("T,dk,dv,seed", [(1, 3, 2, 0), (5, 4, 3, 1), (8, 8, 8, 2), (7, 2, 6, 3)])
def test_brute_force_unrolled(T, dk, dv, seed):
    """Explicit products of the per-token transition matrices (T <= 8, d <= 8)."""
    rng = np.random.default_rng(seed)
    q, k, v, g, beta = _rand_inputs(T, 2, dk, dv, rng, unit=False)
    s0 = rng.standard_normal((2, dk, dv))
    out, sT = oracle_forward(q, k, v, g, beta, 0.7, B=1, T=T, initial_state=s0[None])
    out_u, sT_u = unrolled_np(q, k, v, g, beta, 0.7, s0)
    np.testing.assert_allclose(out, out_u, atol=1e-12, rtol=0)
    np.testing.assert_allclose(sT, sT_u, atol=1e-12, rtol=0)


def test_c_library_matches_numpy_mirror():
    """The C library and the numpy statement of the recurrence agree (fp64, bf16, fp32 in)."""
    rng = np.random.default_rng(7)
    T, H, dk, dv = 37, 3, 16, 8
    q, k, v, g, beta = _rand_inputs(T, H, dk, dv, rng)
    s0 = rng.standard_normal((H, dk, dv))
    for cast in (np.float64, np.float32):
        arrs = [x.astype(cast) for x in (q, k, v, g, beta)]
        out, sT = run(*arrs, 0.3, s0)
        out_n, sT_n = recurrence_np(*arrs, 0.3, s0)
        np.testing.assert_allclose(out, out_n, atol=1e-12)
        np.testing.assert_allclose(sT, sT_n, atol=1e-12)
    # bf16 bit patterns: widening must be exact (truncate fp32 values to bf16 first)
    bits = [(x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
            for x in (q, k, v, g, beta)]
    out, sT = run(*bits, 0.3, s0)
    out_n, sT_n = recurrence_np(*[oracle.widen_np(b) for b in bits], 0.3, s0)
    np.testing.assert_allclose(out, out_n, atol=1e-12)
    np.testing.assert_allclose(sT, sT_n, atol=1e-12)


def test_bf16_widening_exact():
    x = np.array([1.0, -2.5, 3.140625, -5.0, 2.0 ** -100, 0.0], dtype=np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    np.testing.assert_array_equal(oracle.widen_np(bits), x.astype(np.float64))


# ---------------------------------------------------------------- closed forms


def test_orthonormal_keys_no_decay():
    """g = 0 and mutually orthogonal unit keys: every recall is zero, so the state
    is the plain sum of the writes: S_T = sum_t beta_t k_t v_t^T and
    o_t = scale * sum_{s<=t} beta_s (k_s . q_t) v_s."""
    rng = np.random.default_rng(3)
    T, dk, dv = 6, 8, 5
    Q, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Q[:T][:, None, :]
    q = rng.standard_normal((T, 1, dk))
    v = rng.standard_normal((T, 1, dv))
    g = np.zeros((T, 1, dk))
    beta = rng.uniform(0, 1, (T, 1))
    out, sT = run(q, k, v, g, beta, 0.5)
    S = sum(beta[t, 0] * np.outer(k[t, 0], v[t, 0]) for t in range(T))
    np.testing.assert_allclose(sT[0], S, atol=1e-13)
    for t in range(T):
        o = 0.5 * sum(beta[s, 0] * (k[s, 0] @ q[t, 0]) * v[s, 0] for s in range(t + 1))
        np.testing.assert_allclose(out[t, 0], o, atol=1e-13)


def test_channel_aligned_keys_with_decay():
    """Keys on coordinate axes (k_t = e_{c_t}) decouple the state rows: row c_t
    becomes (1 - beta_t) exp(g_t[c_t]) row + beta_t v_t, every other row i just
    decays by exp(g_t[i]).  Checked row by row with a scalar leaky integrator."""
    rng = np.random.default_rng(4)
    T, dk, dv = 20, 5, 3
    chans = rng.integers(0, dk, T)
    k = np.zeros((T, 1, dk))
    k[np.arange(T), 0, chans] = 1.0
    q = rng.standard_normal((T, 1, dk))
    v = rng.standard_normal((T, 1, dv))
    g = rng.uniform(-2.0, 0.0, (T, 1, dk))
    beta = rng.uniform(0, 1, (T, 1))
    s0 = rng.standard_normal((dk, dv))
    out, sT = run(q, k, v, g, beta, 1.0, s0[None])
    rows = [s0[i].copy() for i in range(dk)]
    for t in range(T):
        for i in range(dk):
            rows[i] = rows[i] * np.exp(g[t, 0, i])
        c = chans[t]
        rows[c] = (1.0 - beta[t, 0]) * rows[c] + beta[t, 0] * v[t, 0]
        o = sum(q[t, 0, i] * rows[i] for i in range(dk))
        np.testing.assert_allclose(out[t, 0], o, atol=1e-12)
    np.testing.assert_allclose(sT[0], np.stack(rows), atol=1e-12)


def test_beta_zero_is_pure_cumulative_decay():
    """beta = 0: nothing is written, S_t = Diag(exp(sum_{s<=t} g_s)) S_0 and
    o_t = scale * S_t^T q_t (decay intensity grows with distance)."""
    rng = np.random.default_rng(5)
    T, H, dk, dv = 30, 2, 6, 4
    q, k, v, g, _ = _rand_inputs(T, H, dk, dv, rng)
    beta = np.zeros((T, H))
    s0 = rng.standard_normal((H, dk, dv))
    out, sT = run(q, k, v, g, beta, 0.25, s0)
    G = np.cumsum(g, axis=0)
    for t in range(T):
        St = np.exp(G[t])[:, :, None] * s0
        np.testing.assert_allclose(out[t], 0.25 * np.einsum("hij,hi->hj", St, q[t]), atol=1e-13)
    np.testing.assert_allclose(sT, np.exp(G[-1])[:, :, None] * s0, atol=1e-13)


def test_beta_zero_zero_state_gives_zero():
    rng = np.random.default_rng(6)
    q, k, v, g, _ = _rand_inputs(10, 2, 4, 4, rng)
    out, sT = run(q, k, v, g, np.zeros((10, 2)), 1.0)
    assert np.all(out == 0.0) and np.all(sT == 0.0)


@pytest.mark.parametrize("g_const", [None, 0.0, -5.0])
def test_readback_unit_key_full_write(g_const):
    """beta = 1 and |k| = 1: (I - k k^T) k = 0, so after the write S_t^T k_t = v_t
    exactly, whatever the decay or the earlier state.  With q_t = k_t, scale 1,
    the output is v_t."""
    rng = np.random.default_rng(8)
    T, H, dk, dv = 25, 2, 8, 6
    q, k, v, g, _ = _rand_inputs(T, H, dk, dv, rng)
    if g_const is not None:
        g[:] = g_const
    beta = np.ones((T, H))
    s0 = rng.standard_normal((H, dk, dv))
    out, sT = run(k, k, v, g, beta, 1.0, s0)
    np.testing.assert_allclose(out, v, atol=1e-12)
    np.testing.assert_allclose(np.einsum("hij,hi->hj", sT, k[-1]), v[-1], atol=1e-12)


def test_decay_floor_finite_and_forgets():
    """g = -5 everywhere (the bound): results stay finite, and the initial state's
    influence on o_t shrinks like exp(-5 (t+1)), so two different S_0 agree to
    ~e^-40 relative from t = 7 on."""
    rng = np.random.default_rng(9)
    T, H, dk, dv = 40, 2, 8, 8
    q, k, v, g, beta = _rand_inputs(T, H, dk, dv, rng)
    g[:] = -5.0
    s0a = rng.standard_normal((H, dk, dv)) * 10
    s0b = rng.standard_normal((H, dk, dv)) * 10
    oa, _ = run(q, k, v, g, beta, 1.0, s0a)
    ob, _ = run(q, k, v, g, beta, 1.0, s0b)
    assert np.all(np.isfinite(oa))
    assert np.max(np.abs(oa[7:] - ob[7:])) < 1e-15 * 100
    assert np.max(np.abs(oa[0] - ob[0])) > 1e-4  # the first token still sees S_0


# ---------------------------------------------------------------- invariants


def test_linear_in_values_and_state_jointly_and_in_queries():
    rng = np.random.default_rng(10)
    T, H, dk, dv = 20, 2, 6, 5
    q, k, v1, g, beta = _rand_inputs(T, H, dk, dv, rng)
    v2 = rng.standard_normal(v1.shape)
    s1, s2 = rng.standard_normal((2, H, dk, dv))
    a, b = 0.7, -1.3
    o1, S1 = run(q, k, v1, g, beta, 1.0, s1)
    o2, S2 = run(q, k, v2, g, beta, 1.0, s2)
    o12, S12 = run(q, k, a * v1 + b * v2, g, beta, 1.0, a * s1 + b * s2)
    np.testing.assert_allclose(o12, a * o1 + b * o2, atol=1e-12)
    np.testing.assert_allclose(S12, a * S1 + b * S2, atol=1e-12)
    q2 = rng.standard_normal(q.shape)
    oq1, _ = run(q, k, v1, g, beta, 1.0, s1)
    oq2, _ = run(q2, k, v1, g, beta, 1.0, s1)
    oq12, _ = run(a * q + b * q2, k, v1, g, beta, 1.0, s1)
    np.testing.assert_allclose(oq12, a * oq1 + b * oq2, atol=1e-12)


@pytest.mark.parametrize("split", [1, 17, 39])
def test_split_sequence_state_passing(split):
    """Prefix caching: running [0, T1) then [T1, T) from the returned state equals
    one run (best.xiaohu.ai, section "Infrastructure efficiency": KDA state
    snapshots at segment boundaries; neurohive.io, section "Training and
    inference infrastructure": one state copy per request)."""
    rng = np.random.default_rng(11)
    T, H, dk, dv = 40, 2, 6, 5
    q, k, v, g, beta = _rand_inputs(T, H, dk, dv, rng)
    s0 = rng.standard_normal((H, dk, dv))
    o, S = run(q, k, v, g, beta, 0.5, s0)
    oa, Sa = run(q[:split], k[:split], v[:split], g[:split], beta[:split], 0.5, s0)
    ob, Sb = run(q[split:], k[split:], v[split:], g[split:], beta[split:], 0.5, Sa)
    np.testing.assert_allclose(np.concatenate([oa, ob]), o, atol=1e-12)
    np.testing.assert_allclose(Sb, S, atol=1e-12)


def test_state_norm_never_grows_without_values():
    """v = 0, g <= 0, beta in [0,1], |k| = 1: each factor (I - beta k k^T) and
    Diag(exp g) has norm <= 1, so the Frobenius norm of S never increases."""
    rng = np.random.default_rng(12)
    T, dk, dv = 30, 6, 4
    q, k, _, g, beta = _rand_inputs(T, 1, dk, dv, rng, g_lo=-0.3)
    v = np.zeros((T, 1, dv))
    S = rng.standard_normal((1, dk, dv))
    prev = np.linalg.norm(S)
    for t in range(T):
        _, S = run(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], beta[t:t + 1], 1.0, S)
        now = np.linalg.norm(S)
        assert now <= prev * (1 + 1e-14)
        prev = now


def test_state_size_independent_of_length():
    """Fixed-size memory: the state is dk x dv whether T is 3 or 300."""
    rng = np.random.default_rng(13)
    for T in (3, 300):
        q, k, v, g, beta = _rand_inputs(T, 2, 8, 4, rng)
        _, S = run(q, k, v, g, beta)
        assert S.shape == (2, 8, 4)


def test_varlen_equals_separate_sequences():
    rng = np.random.default_rng(14)
    lens = [5, 1, 17, 9]
    H, dk, dv = 2, 4, 3
    q, k, v, g, beta = _rand_inputs(sum(lens), H, dk, dv, rng)
    s0 = rng.standard_normal((len(lens), H, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lens)])
    out, sT = oracle_forward(q, k, v, g, beta, 0.9, cu_seqlens=cu, initial_state=s0)
    for n in range(len(lens)):
        sl = slice(cu[n], cu[n + 1])
        o, S = run(q[sl], k[sl], v[sl], g[sl], beta[sl], 0.9, s0[n])
        np.testing.assert_allclose(out[sl], o, atol=1e-13)
        np.testing.assert_allclose(sT[n * H:(n + 1) * H], S, atol=1e-13)


def test_pair_subset_and_packed_output():
    rng = np.random.default_rng(15)
    lens = [6, 11]
    H, dk, dv = 3, 4, 2
    q, k, v, g, beta = _rand_inputs(sum(lens), H, dk, dv, rng)
    cu = np.concatenate([[0], np.cumsum(lens)])
    full, sfull = oracle_forward(q, k, v, g, beta, 1.0, cu_seqlens=cu)
    pieces, sp = oracle_forward(q, k, v, g, beta, 1.0, cu_seqlens=cu, pairs=[(1, 2), (0, 1)],
                                packed=True)
    np.testing.assert_array_equal(pieces[0], full[cu[1]:cu[2], 2])
    np.testing.assert_array_equal(pieces[1], full[cu[0]:cu[1], 1])
    np.testing.assert_array_equal(sp[0], sfull[1 * H + 2])
    np.testing.assert_array_equal(sp[1], sfull[0 * H + 1])


# ---------------------------------------------------------------- chunked algebra


@pytest.mark.parametrize("C", [1, 16, 64, 1000])
@pytest.mark.parametrize("g_lo", [-5.0, -0.05])
def test_chunked_form_matches_recurrence(C, g_lo):
    """The chunked algebra the GPU prefill is built on equals the recurrence for
    every chunk size (chunk-size invariance), with ragged last chunks."""
    rng = np.random.default_rng(16)
    T, H, dk, dv = 150, 2, 16, 8
    q, k, v, g, beta = _rand_inputs(T, H, dk, dv, rng, g_lo=g_lo)
    s0 = rng.standard_normal((H, dk, dv))
    o, S = run(q, k, v, g, beta, 0.3, s0)
    oc, Sc = cf.chunked_forward(q, k, v, g, beta, 0.3, C=C, initial_state=s0)
    np.testing.assert_allclose(oc, o, atol=1e-11)
    np.testing.assert_allclose(Sc, S, atol=1e-11)


def test_subtile_factors_bounded_at_decay_floor():
    """With log-decay >= -5, 16-row sub-tiles referenced to their own end keep
    every factor in [e^-80, e^80] (inside bf16/fp32 range: ln(max) ~ 88.7), and the
    factored Gram equals the direct one.  Over a whole 64-row chunk the direct
    factor exp(-G) would reach e^320 and overflow fp32."""
    rng = np.random.default_rng(17)
    n, dk = 64, 8
    g = np.full((n, dk), -5.0)
    g[:, 0] = rng.uniform(-5, 0, n)
    a = rng.standard_normal((n, dk))
    b = rng.standard_normal((n, dk))
    f = cf.subtile_factors(g)
    for key in ("rowf", "colf"):
        assert np.all(f[key] <= np.exp(80.0) * (1 + 1e-12))
        assert np.all(f[key] >= np.exp(-80.0) * (1 - 1e-12))
    assert all(np.all(p <= 1.0) for p in f["pair"].values())
    G = np.cumsum(g, axis=0)
    assert np.max(-G) > 88.8  # the unfactored reciprocal overflows fp32
    direct = np.tril(np.einsum("tc,sc,tsc->ts", a, b,
                               np.exp(np.minimum(G[:, None, :] - G[None, :, :], 0.0))))
    np.testing.assert_allclose(cf.gram_from_subtiles(a, b, g), direct, atol=1e-12, rtol=1e-12)


# ---------------------------------------------------------------- planted mistakes


def _mutant(kind):
    """A copy of the recurrence with one plausible mistake planted."""
    def fwd(q, k, v, g, beta, scale, s0=None):
        T, H, dk = q.shape
        dv = v.shape[-1]
        S = np.zeros((H, dk, dv)) if s0 is None else s0.copy()
        out = np.zeros((T, H, dv))
        for t in range(T):
            d = np.exp(g[t])
            if kind == "decay_after_write":
                pass
            elif kind == "decay_on_columns":
                S = S * d[:, None, :dv] if dk >= dv else S
            else:
                S = S * d[:, :, None]
            recall = np.einsum("hij,hi->hj", S, k[t])
            w = beta[t][:, None] * (v[t] - recall)
            if kind == "sign_flip":
                w = beta[t][:, None] * (v[t] + recall)
            if kind == "read_before_write":
                out[t] = np.einsum("hij,hi->hj", S, scale * q[t])
            S = S + k[t][:, :, None] * w[:, None, :]
            if kind == "decay_after_write":
                S = S * d[:, :, None]
            if kind != "read_before_write":
                out[t] = np.einsum("hij,hi->hj", S, scale * q[t])
        return out, S
    return fwd


@pytest.mark.parametrize("kind", ["decay_after_write", "decay_on_columns", "sign_flip",
                                  "read_before_write"])
def test_pins_catch_planted_mistakes(kind):
    """Each planted mistake fails the hand-worked example or a closed form."""
    fwd = _mutant(kind)
    failures = 0
    d = _read_golden("handworked_2x2.txt")
    q = np.stack([d["q1"], d["q2"]])[:, None, :]
    k = np.stack([d["k1"], d["k2"]])[:, None, :]
    v = np.stack([d["v1"], d["v2"]])[:, None, :]
    g = np.stack([d["g1"], d["g2"]])[:, None, :]
    beta = np.array([d["beta1"][0], d["beta2"][0]])[:, None]
    out, S = fwd(q, k, v, g, beta, 1.0, d["S0"].reshape(1, 2, 2))
    failures += not np.allclose(out[1, 0], d["o2"], atol=1e-9)
    # read-back closed form
    rng = np.random.default_rng(18)
    q, k, v, g, _ = _rand_inputs(10, 1, 4, 4, rng)
    out, _ = fwd(k, k, v, g, np.ones((10, 1)), 1.0, rng.standard_normal((1, 4, 4)))
    failures += not np.allclose(out, v, atol=1e-9)
    assert failures >= 1


# ---------------------------------------------------------------- prologue


def test_prologue_against_library_routines():
    """q, k: same direction as the input with unit norm (torch's normalize, where the
    norm dwarfs the epsilon); g: torch's softplus with the -5 clamp; beta: sigmoid."""
    import torch
    from oracle import prologue_np
    rng = np.random.default_rng(40)
    q, k, g, b = (rng.standard_normal(s) * 2.0 for s in ((7, 3, 16), (7, 3, 16), (7, 3, 16), (7, 3)))
    qn, kn, gg, bb = prologue_np(q, k, g, b)
    tq = torch.nn.functional.normalize(torch.tensor(q), dim=-1).numpy()
    tk = torch.nn.functional.normalize(torch.tensor(k), dim=-1).numpy()
    np.testing.assert_allclose(qn, tq, rtol=1e-6, atol=0)
    np.testing.assert_allclose(kn, tk, rtol=1e-6, atol=0)
    np.testing.assert_allclose(np.linalg.norm(qn, axis=-1), 1.0, rtol=1e-6)
    tg = torch.clamp(-torch.nn.functional.softplus(torch.tensor(g)), min=-5.0).numpy()
    np.testing.assert_allclose(gg, tg, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(bb, torch.sigmoid(torch.tensor(b)).numpy(), rtol=1e-14, atol=0)


def test_prologue_special_values():
    from oracle import prologue_np
    x = np.array([0.0, 100.0, -100.0, np.log(np.expm1(5.0)), 3.0])
    _, _, g, b = prologue_np(np.ones((1, 2)), np.ones((1, 2)), x, x)
    assert g[0] == pytest.approx(-np.log(2.0), abs=1e-15)     # softplus(0) = ln 2
    assert g[1] == -5.0                                         # clamped at the floor
    assert -1e-40 < g[2] <= 0.0                                 # retention -> 1
    assert g[3] == pytest.approx(-5.0, abs=1e-12)               # exactly at the floor
    assert b[0] == 0.5 and b[1] == 1.0 and b[2] < 1e-40
    assert b[4] == pytest.approx(1.0 - b[4] * np.exp(-3.0), abs=1e-15)   # beta = 1/(1+e^-x)
    # a zero vector stays zero instead of dividing by zero
    qn, _, _, _ = prologue_np(np.zeros((1, 4)), np.ones((1, 4)), x[:1], x[:1])
    assert np.all(qn == 0.0)


# ---------------------------------------------------------------- backward


def _loss_fd_setup(seed, T=7, H=2, dk=3, dv=2):
    rng = np.random.default_rng(seed)
    q, k, v, g, beta = _rand_inputs(T, H, dk, dv, rng, beta_lo=0.05, beta_hi=0.95)
    s0 = rng.standard_normal((H, dk, dv)) * 0.3
    d_out = rng.standard_normal((T, H, dv))
    d_fin = rng.standard_normal((H, dk, dv))
    return dict(q=q, k=k, v=v, g=g, beta=beta, s0=s0), d_out, d_fin


def _loss(x, d_out, d_fin, scale):
    out, sT = run(x["q"], x["k"], x["v"], x["g"], x["beta"], scale, x["s0"])
    return float((out * d_out).sum() + (sT.reshape(d_fin.shape) * d_fin).sum())


@pytest.mark.parametrize("seed", [50, 51])
def test_backward_matches_finite_differences(seed):
    """Every gradient of the autodiff oracle equals the central finite difference of
    the C oracle's forward loss (a separate implementation of the recurrence),
    element by element: error O(h^2) + rounding, well under 1e-7 relative."""
    from oracle import backward_oracle
    x, d_out, d_fin = _loss_fd_setup(seed)
    scale = 0.7
    gr = backward_oracle(x["q"][None], x["k"][None], x["v"][None], x["g"][None],
                         x["beta"][None], scale, d_out[None], x["s0"][None], d_fin[None])
    names = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", s0="ds0")
    h = 1e-5
    for name, key in names.items():
        got = gr[key][0]
        fd = np.zeros_like(x[name])
        for idx in np.ndindex(*x[name].shape):
            xp = {kk: vv.copy() for kk, vv in x.items()}
            xm = {kk: vv.copy() for kk, vv in x.items()}
            xp[name][idx] += h
            xm[name][idx] -= h
            fd[idx] = (_loss(xp, d_out, d_fin, scale) - _loss(xm, d_out, d_fin, scale)) / (2 * h)
        err = np.max(np.abs(got - fd)) / max(1.0, np.max(np.abs(fd)))
        assert err < 1e-7, f"d{name}: {err:.3e}"


def test_backward_beta_zero_closed_form():
    """With beta = 0 nothing is written: S_t = Diag(exp G_t) S_0 with G_t the running
    sum of g, so o_t = scale S_t^T q_t.  Then dk = dv = 0 exactly,
    dq_t = scale Diag(exp G_t) S_0 dO_t, dS_0 = sum_t scale exp(G_t) * q_t dO_t^T +
    exp(G_T) * dS_T (products with exp per row), and dg_t = sum over u >= t of the
    row-wise terms of <dS_u, ...>, checked here through dg_t = sum_{u>=t} r_u with
    r_u = scale q_u * (S_u dO_u) and the final-state term on the last token."""
    from oracle import backward_oracle
    rng = np.random.default_rng(52)
    T, H, dk, dv, scale = 6, 2, 4, 3, 0.9
    q, k, v, g, _ = _rand_inputs(T, H, dk, dv, rng)
    beta = np.zeros((T, H))
    s0 = rng.standard_normal((H, dk, dv))
    d_out = rng.standard_normal((T, H, dv))
    d_fin = rng.standard_normal((H, dk, dv))
    gr = backward_oracle(q[None], k[None], v[None], g[None], beta[None], scale, d_out[None],
                         s0[None], d_fin[None])
    assert np.all(gr["dk"] == 0.0) and np.all(gr["dv"] == 0.0)
    G = np.cumsum(g, axis=0)                                   # [T, H, dk]
    St = np.exp(G)[..., None] * s0[None]                       # [T, H, dk, dv]
    dq = scale * np.einsum("thij,thj->thi", St, d_out)
    np.testing.assert_allclose(gr["dq"][0], dq, rtol=1e-12, atol=1e-12)
    ds0 = (scale * np.exp(G)[..., None] * q[..., None] * d_out[:, :, None, :]).sum(0) \
        + np.exp(G[-1])[..., None] * d_fin
    np.testing.assert_allclose(gr["ds0"][0], ds0, rtol=1e-12, atol=1e-12)
    r = scale * q * np.einsum("thij,thj->thi", St, d_out)      # d<dO_u, o_u>/dG_u
    r[-1] += np.einsum("hij,hij->hi", St[-1], d_fin)           # final-state term
    dg = np.cumsum(r[::-1], axis=0)[::-1]
    np.testing.assert_allclose(gr["dg"][0], dg, rtol=1e-12, atol=1e-12)
    # dbeta: d<...>/dbeta_t with nothing written = <k_t (v_t - S_t^T k_t)^T, cotangent of S_t>
    assert np.all(np.isfinite(gr["dbeta"]))


@pytest.mark.parametrize("kind", ["sign_flip", "decay_after_write"])
def test_backward_pins_catch_planted_mistakes(kind, monkeypatch):
    """A plausible mistake planted in the autodiff oracle's recurrence makes its
    gradients disagree with the finite differences of the C oracle."""
    import torch
    from oracle import backward_oracle, grad

    def mutant(q, k, v, g, beta, scale, s0):
        S, outs = s0, []
        for t in range(q.shape[1]):
            d = torch.exp(g[:, t])[:, :, None]
            if kind != "decay_after_write":
                S = S * d
            recall = (S * k[:, t, :, None]).sum(1)
            sgn = 1.0 if kind == "sign_flip" else -1.0
            write = beta[:, t, None] * (v[:, t] + sgn * recall)
            S = S + k[:, t, :, None] * write[:, None, :]
            if kind == "decay_after_write":
                S = S * d
            outs.append((S * (scale * q[:, t, :, None])).sum(1))
        return torch.stack(outs, 1), S

    monkeypatch.setattr(grad, "_recurrence", mutant)
    x, d_out, d_fin = _loss_fd_setup(53)
    gr = backward_oracle(x["q"][None], x["k"][None], x["v"][None], x["g"][None],
                         x["beta"][None], 0.7, d_out[None], x["s0"][None], d_fin[None])
    h, idx = 1e-5, (3, 1, 2)
    xp = {kk: vv.copy() for kk, vv in x.items()}
    xm = {kk: vv.copy() for kk, vv in x.items()}
    xp["k"][idx] += h
    xm["k"][idx] -= h
    fd = (_loss(xp, d_out, d_fin, 0.7) - _loss(xm, d_out, d_fin, 0.7)) / (2 * h)
    assert abs(gr["dk"][0][idx] - fd) > 1e-4


# ---------------------------------------------------------------- transition (context parallelism)


def test_transition_is_the_linear_part_of_the_c_oracle():
    """The C oracle's exit state is affine in the entry state: S_T(S0) - S_T(0) = P S0
    with P from transition_np, for random entry states (a separate implementation of
    the recurrence on each side)."""
    from oracle import transition_np
    rng = np.random.default_rng(60)
    T, H, dk, dv = 23, 2, 6, 5
    q, k, v, g, beta = _rand_inputs(T, H, dk, dv, rng)
    P = transition_np(k, g, beta)
    _, s_zero = run(q, k, v, g, beta, 0.5, np.zeros((H, dk, dv)))
    for _ in range(2):
        s0 = rng.standard_normal((H, dk, dv))
        _, s_t = run(q, k, v, g, beta, 0.5, s0)
        np.testing.assert_allclose(s_t.reshape(H, dk, dv) - s_zero.reshape(H, dk, dv),
                                   np.einsum("hij,hjk->hik", P, s0), rtol=1e-10, atol=1e-12)


def test_transition_special_cases():
    """beta = 0: pure decay, P = Diag(exp(sum g)).  One token with g = 0, beta = 1 and
    a unit key: the projector I - k k^T (P k = 0, P^2 = P).  Segments compose: the
    transition of a concatenation is the later transition times the earlier one."""
    from oracle import transition_np
    rng = np.random.default_rng(61)
    T, H, dk = 9, 2, 5
    _, k, _, g, _ = _rand_inputs(T, H, dk, 3, rng)
    P = transition_np(k, g, np.zeros((T, H)))
    for h in range(H):
        np.testing.assert_allclose(P[h], np.diag(np.exp(g[:, h].sum(0))), rtol=1e-13, atol=0)
    P1 = transition_np(k[:1], np.zeros((1, H, dk)), np.ones((1, H)))
    for h in range(H):
        np.testing.assert_allclose(P1[h] @ k[0, h], 0.0, atol=1e-14)
        np.testing.assert_allclose(P1[h] @ P1[h], P1[h], atol=1e-14)
    beta = rng.uniform(0, 1, (T, H))
    Pa, Pb, Pab = transition_np(k[:4], g[:4], beta[:4]), transition_np(k[4:], g[4:], beta[4:]), \
        transition_np(k, g, beta)
    np.testing.assert_allclose(Pab, np.einsum("hij,hjk->hik", Pb, Pa), rtol=1e-12, atol=1e-14)
