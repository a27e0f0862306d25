"""GPU parity of the fused prefill (bf16, d = 128, 256 or more (sequence, head)
streams: one workgroup per stream, chunk operands kept on chip), through the C ABI,
against the fp64 oracle: packed sequences with empty, one-token, exact-chunk and
ragged lengths; fixed length; both ends of the decay range; nonzero and absent
initial states; the state updated in place; no final state.  Tolerances of
tests/parity.py (bf16: max-abs <= 2e-2, rel-L2 <= 1e-2, whole tensors)."""
import math

import numpy as np
import pytest
import torch

from gated_delta_rule_102_amd import inputs as kin
from oracle import oracle_forward
from tests.parity import assert_close, oracle_fixed

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    from gated_delta_rule_102_amd import kda
    kda.load_library()
    torch.cuda.set_device(0)
    yield


def _dev(d):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def test_fused_schedule_is_selected():
    from gated_delta_rule_102_amd import kda
    assert kda.prefill_schedule_name(16, 0, 16, 128, varlen=True, total_T=1000).startswith("fused")
    assert kda.prefill_schedule_name(2, 150, 128, 128).startswith("fused")
    assert not kda.prefill_schedule_name(2, 150, 64, 128).startswith("fused")


@pytest.mark.parametrize("with_state", [True, False])
def test_fused_varlen_ragged(with_state):
    from gated_delta_rule_102_amd import kda
    lengths = [0, 1, 63, 64, 65, 130, 300, 5, 17, 200, 128, 1, 77, 256, 31, 90]
    H, D = 16, 128
    d = kin.make_varlen(lengths, H, D, D, seed=61, nonzero_state=with_state, split_decay=True)
    d["scale"] = 1.0 / math.sqrt(D)
    g = _dev(d)
    out, fs = kda.kda_chunk_fwd_varlen(g["q"], g["k"], g["v"], g["g"], g["beta"], g["cu_seqlens"],
                                       d["scale"], initial_state=g["initial_state"])
    torch.cuda.synchronize()
    ref_o, ref_s = oracle_forward(d["q"][0], d["k"][0], d["v"][0], d["g"][0], d["beta"][0],
                                  d["scale"], cu_seqlens=d["cu_seqlens"].numpy(),
                                  initial_state=d["initial_state"])
    assert_close("fused varlen out", out[0], ref_o, torch.bfloat16)
    assert_close("fused varlen state", fs, ref_s.reshape(fs.shape), torch.bfloat16)
    # the empty sequence's final state is its initial state (or zero)
    s0 = d["initial_state"][0] if with_state else torch.zeros(H, D, D)
    assert torch.equal(fs[0].cpu(), s0)


@pytest.mark.parametrize("B,T,H", [(2, 150, 128), (1, 320, 256), (4, 64, 64)])
def test_fused_fixed_length(B, T, H):
    d = kin.make_prefill(B, T, H, 128, 128, seed=70 + T, nonzero_state=True)
    d["scale"] = 1.0 / math.sqrt(128)
    from gated_delta_rule_102_amd import kda
    g = _dev(d)
    out, fs = kda.kda_chunk_fwd(g["q"], g["k"], g["v"], g["g"], g["beta"], d["scale"],
                                g["initial_state"])
    torch.cuda.synchronize()
    ref_o, ref_s = oracle_fixed(d)
    assert_close(f"fused {B}x{T}x{H} out", out, ref_o.reshape(out.shape), torch.bfloat16)
    assert_close(f"fused {B}x{T}x{H} state", fs, ref_s.reshape(fs.shape), torch.bfloat16)


@pytest.mark.parametrize("B,T,H,with_state", [(1, 8200, 32, True),    # 8 segments, 8-token tail
                                               (1, 16400, 16, True),   # 16 segments
                                               (3, 11000, 8, True),    # 10 unequal segments
                                               (1, 32800, 4, False)])  # 32 segments
def test_fused_segmented(B, T, H, with_state):
    """Few long sequences: each cut into segments whose exit states and transitions
    compose into every segment's entry state before the outputs run."""
    from gated_delta_rule_102_amd import kda
    assert "segments" in kda.prefill_schedule_name(B, T, H, 128)
    d = kin.make_prefill(B, T, H, 128, 128, seed=80 + T + H, nonzero_state=with_state)
    d["scale"] = 1.0 / math.sqrt(128)
    g = _dev(d)
    args = [g[x] for x in ("q", "k", "v", "g", "beta")]
    out, fs = kda.kda_chunk_fwd(*args, d["scale"], g.get("initial_state"))
    torch.cuda.synchronize()
    ref_o, ref_s = oracle_fixed(d)
    assert_close(f"segmented {B}x{T}x{H} out", out, ref_o.reshape(out.shape), torch.bfloat16)
    assert_close(f"segmented {B}x{T}x{H} state", fs, ref_s.reshape(fs.shape), torch.bfloat16)
    if with_state:   # the final state may overwrite the initial state
        st = g["initial_state"].clone()
        out2, _ = kda.kda_chunk_fwd(*args, d["scale"], st, final_state=st)
        torch.cuda.synchronize()
        assert torch.equal(out, out2) and torch.equal(fs, st)
    # on a caller workspace of exactly the stated size, and without a final state:
    # the same outputs bit for bit
    ws = kda.chunk_fwd_workspace(g["q"], g["v"])
    assert ws.numel() - 256 == kda.kda_chunk_fwd_workspace_size(B, T, H, 128, 128)
    out3, fs3 = kda.kda_chunk_fwd(*args, d["scale"], g.get("initial_state"), workspace=ws)
    out4, none = kda.kda_chunk_fwd(*args, d["scale"], g.get("initial_state"),
                                   output_final_state=False)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(out, out3) and torch.equal(fs, fs3) and torch.equal(out, out4)


@pytest.mark.parametrize("mode", ["floor", "slow", "zero"])
def test_fused_decay_extremes(mode):
    """g = -5 everywhere (sub-tile factors reach e^75, the chunk's e^-320 underflows),
    g in [-0.05, 0] (almost no forgetting) and g = 0 (plain delta rule)."""
    from gated_delta_rule_102_amd import kda
    d = kin.make_prefill(2, 200, 128, 128, 128, seed=81, nonzero_state=True)
    if mode == "floor":
        d["g"] = torch.full_like(d["g"], -5.0)
    elif mode == "slow":
        d["g"] = (-0.05 * torch.rand(d["g"].shape, generator=torch.Generator().manual_seed(4))
                  ).to(torch.bfloat16)
    else:
        d["g"] = torch.zeros_like(d["g"])
    d["scale"] = 1.0 / math.sqrt(128)
    g = _dev(d)
    out, fs = kda.kda_chunk_fwd(g["q"], g["k"], g["v"], g["g"], g["beta"], d["scale"],
                                g["initial_state"])
    torch.cuda.synchronize()
    ref_o, ref_s = oracle_fixed(d)
    assert_close(f"fused decay {mode} out", out, ref_o.reshape(out.shape), torch.bfloat16)
    assert_close(f"fused decay {mode} state", fs, ref_s.reshape(fs.shape), torch.bfloat16)


@pytest.mark.parametrize("mode", ["floor", "slow", "zero"])
def test_fused_segmented_decay_extremes(mode):
    """The segmented schedule where the segments' transitions matter most: g = 0
    (plain delta rule, the transitions do not decay) and g in [-0.05, 0], and at the
    floor g = -5 (the transitions underflow to zero), 16 segments of 16 chunks, with
    an initial state."""
    from gated_delta_rule_102_amd import kda
    B, T, H = 1, 16400, 16
    assert "in 16 segments" in kda.prefill_schedule_name(B, T, H, 128)
    d = kin.make_prefill(B, T, H, 128, 128, seed=83, nonzero_state=True)
    if mode == "floor":
        d["g"] = torch.full_like(d["g"], -5.0)
    elif mode == "slow":
        d["g"] = (-0.05 * torch.rand(d["g"].shape, generator=torch.Generator().manual_seed(5))
                  ).to(torch.bfloat16)
    else:
        d["g"] = torch.zeros_like(d["g"])
    d["scale"] = 1.0 / math.sqrt(128)
    g = _dev(d)
    out, fs = kda.kda_chunk_fwd(g["q"], g["k"], g["v"], g["g"], g["beta"], d["scale"],
                                g["initial_state"])
    torch.cuda.synchronize()
    ref_o, ref_s = oracle_fixed(d)
    eo = assert_close(f"segmented decay {mode} out", out, ref_o.reshape(out.shape), torch.bfloat16)
    es = assert_close(f"segmented decay {mode} state", fs, ref_s.reshape(fs.shape), torch.bfloat16)
    print(f"segmented decay {mode}: out max_abs {eo[0]:.2e} rel_l2 {eo[1]:.2e}; "
          f"state max_abs {es[0]:.2e} rel_l2 {es[1]:.2e}", flush=True)


def test_fused_in_place_and_no_final_state():
    from gated_delta_rule_102_amd import kda
    d = _dev(kin.make_prefill(2, 130, 128, 128, 128, seed=91, nonzero_state=True))
    sc = 1.0 / math.sqrt(128)
    out, fs = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], sc, d["initial_state"])
    st = d["initial_state"].clone()
    out2, _ = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], sc, st, final_state=st)
    out3, none = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], sc,
                                   d["initial_state"], output_final_state=False)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(out, out2) and torch.equal(out, out3) and torch.equal(fs, st)


def test_fused_deterministic_and_equal_to_separate_calls():
    """Run to run bitwise equal; each packed sequence equals its own fixed-length call
    with the same head count (also fused, same kernel)."""
    from gated_delta_rule_102_amd import kda
    lengths = [70, 3, 129, 256]
    H = 64
    d = _dev(kin.make_varlen(lengths, H, 128, 128, seed=93, nonzero_state=True))
    sc = 1.0 / math.sqrt(128)
    args = [d[x] for x in ("q", "k", "v", "g", "beta")]
    o1, s1 = kda.kda_chunk_fwd_varlen(*args, d["cu_seqlens"], sc, initial_state=d["initial_state"])
    o2, s2 = kda.kda_chunk_fwd_varlen(*args, d["cu_seqlens"], sc, initial_state=d["initial_state"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    cu = d["cu_seqlens"].tolist()
    rows = []
    for n, L in enumerate(lengths):
        sl = slice(cu[n], cu[n + 1])
        # repeat the sequence 4 times so the fixed-length call has 256 streams
        rep = [x[:, sl].expand(4, -1, -1, -1).contiguous() if x.dim() == 4 else
               x[:, sl].expand(4, -1, -1).contiguous() for x in args]
        s0 = d["initial_state"][n:n + 1].expand(4, -1, -1, -1).contiguous()
        o, s = kda.kda_chunk_fwd(*rep, sc, s0)
        torch.cuda.synchronize()
        assert torch.equal(o[0], o1[0, sl]), f"sequence {n}: output differs from its own call"
        assert torch.equal(s[0], s1[n]), f"sequence {n}: state differs from its own call"
        rows.append(n)
    assert rows == list(range(len(lengths)))
