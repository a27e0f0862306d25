"""fp32 prefill at dk = dv = 128 (kda_chunk_fwd / kda_chunk_fwd_varlen, through the C
ABI), which runs on fp32 chunk operands in windows of chunks: outputs and final states
against the fp64 oracle at the fp32 tolerance (rel-L2 <= 1e-4) -- one window and
several (17 and 40 chunks with 16-chunk windows), a ragged tail, no initial state,
the state updated in place, packed sequences (empty, one token, longer than a window)
-- and the caller-workspace form with a workspace sized for one-chunk windows bit for
bit equal to the default windows, as is the allocation-free form."""
import math

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


@pytest.mark.parametrize("B,T,H,state", [(2, 150, 3, True), (1, 1088, 2, True),
                                         (1, 2560, 1, False), (3, 64, 2, True)])
def test_fp32_d128_fixed_matches_oracle(B, T, H, state):
    from gated_delta_rule_102_amd import kda
    d = kin.make_prefill(B, T, H, 128, 128, dtype=torch.float32, seed=600 + T, nonzero_state=state)
    d["scale"] = 1.0 / math.sqrt(128)
    assert kda.prefill_schedule_name(B, T, H, 128, torch.float32).startswith("chunk_ops_kernel<128,f32>")
    g = _dev(d)
    out, fs = kda.kda_chunk_fwd(g["q"], g["k"], g["v"], g["g"], g["beta"], d["scale"],
                                g.get("initial_state"))
    torch.cuda.synchronize()
    ref_o, ref_s = oracle_fixed(d)
    assert_close(f"fp32 d128 {B}x{T}x{H} out", out, ref_o.reshape(out.shape), torch.float32)
    assert_close(f"fp32 d128 {B}x{T}x{H} state", fs, ref_s.reshape(fs.shape), torch.float32)


def test_fp32_d128_in_place_workspace_and_noalloc():
    from gated_delta_rule_102_amd import kda
    B, T, H = 2, 700, 2
    d = _dev(kin.make_prefill(B, T, H, 128, 128, dtype=torch.float32, seed=650, nonzero_state=True))
    sc = 1.0 / math.sqrt(128)
    args = [d[x] for x in ("q", "k", "v", "g", "beta")]
    ref_o, ref_s = kda.kda_chunk_fwd(*args, sc, d["initial_state"])
    st = d["initial_state"].clone()
    o2, _ = kda.kda_chunk_fwd(*args, sc, st, final_state=st)
    # a workspace that holds one-chunk windows only: the same arithmetic in more windows
    small = kda.load_library().kda_chunk_fwd_workspace_size(1, 64, B * H, 128, 128, 1)
    ws = torch.empty(small + 256, dtype=torch.uint8, device=DEV)
    ws.fill_(0x77)
    o3, s3 = kda.kda_chunk_fwd(*args, sc, d["initial_state"], workspace=ws)
    o4, s4 = kda.kda_chunk_fwd_noalloc(*args, sc, d["initial_state"])
    torch.cuda.synchronize()
    assert torch.equal(o2, ref_o) and torch.equal(st, ref_s), "in place"
    assert torch.equal(o3, ref_o) and torch.equal(s3, ref_s), "one-chunk windows"
    assert torch.equal(o4, ref_o) and torch.equal(s4, ref_s), "allocation-free form"


def test_fp32_d128_varlen_matches_oracle():
    from gated_delta_rule_102_amd import kda
    lengths = [70, 0, 1, 1100, 129]
    H = 2
    d = kin.make_varlen(lengths, H, 128, 128, dtype=torch.float32, seed=660, nonzero_state=True)
    d["scale"] = 1.0 / math.sqrt(128)
    g = _dev(d)
    out, fs = kda.kda_chunk_fwd_varlen(g["q"], g["k"], g["v"], g["g"], g["beta"], g["cu_seqlens"],
                                       d["scale"], initial_state=g["initial_state"])
    torch.cuda.synchronize()
    ref_o, ref_s = oracle_forward(d["q"][0], d["k"][0], d["v"][0], d["g"][0], d["beta"][0],
                                  d["scale"], cu_seqlens=d["cu_seqlens"].numpy(),
                                  initial_state=d["initial_state"])
    assert_close("fp32 d128 varlen out", out[0], ref_o, torch.float32)
    assert_close("fp32 d128 varlen state", fs, ref_s.reshape(fs.shape), torch.float32)
    assert torch.equal(fs[1].cpu(), d["initial_state"][1]), "empty sequence: state passes through"
