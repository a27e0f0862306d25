"""The backward in windows of chunks (kda_chunk_bwd_ws / kda_chunk_bwd_varlen_ws given
less workspace than the one-pass size, through the C ABI): every gradient and the
initial-state gradient bit for bit equal to the one-pass call's -- the windowed form
runs the same per-chunk arithmetic, with the states and state gradients at window
boundaries passed through memory in fp32 -- for fixed length (last window partial, one
chunk per window, a ragged tail) and for packed sequences (empty, shorter than a
window, spanning several), bf16 and fp32; plus one windowed call against the fp64
autodiff oracle directly."""
import math

import pytest
import torch

from gated_delta_rule_102_amd import inputs as kin
from oracle import backward_oracle
from tests.test_gpu_backward import NAMES, grad_close

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


@pytest.mark.parametrize("dtype,D,B,T,H,cw", [(torch.bfloat16, 128, 2, 300, 3, 2),
                                              (torch.bfloat16, 128, 1, 200, 2, 1),
                                              (torch.float32, 128, 2, 260, 2, 3),
                                              (torch.bfloat16, 64, 1, 450, 4, 2),
                                              (torch.float32, 64, 3, 130, 2, 1)])
def test_windowed_backward_equals_one_pass(dtype, D, B, T, H, cw):
    from gated_delta_rule_102_amd import kda
    d = _dev(kin.make_prefill(B, T, H, D, D, dtype=dtype, seed=500 + T + cw, nonzero_state=True))
    c = _dev(kin.make_cotangents(B, T, H, D, D, dtype=dtype, seed=510 + T))
    sc = 1.0 / math.sqrt(D)
    args = [d[x] for x in ("q", "k", "v", "g", "beta")]
    full = kda.kda_chunk_bwd(*args, c["grad_out"], sc, d["initial_state"], c["grad_final_state"])
    ws = kda.chunk_bwd_workspace(d["q"], d["v"], window_chunks=cw)
    assert ws.numel() < kda.chunk_bwd_workspace(d["q"], d["v"]).numel()
    ws.fill_(0x5A)
    for rep in range(2):
        got = kda.kda_chunk_bwd(*args, c["grad_out"], sc, d["initial_state"], c["grad_final_state"],
                                workspace=ws)
        torch.cuda.synchronize()
        for n, x, y in zip(NAMES, got, full):
            assert torch.equal(x, y), f"rep {rep} {n}: windowed != one pass"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_windowed_varlen_backward_equals_one_pass(dtype):
    from gated_delta_rule_102_amd import kda
    lengths = [70, 0, 129, 260, 3, 64]
    H, D = 2, 128
    d = _dev(kin.make_varlen(lengths, H, D, D, dtype=dtype, seed=520, nonzero_state=True))
    total = sum(lengths)
    c = kin.make_cotangents(1, total, H, D, D, dtype=dtype, seed=521, final_state=False)
    dsT = torch.randn((len(lengths), H, D, D), generator=torch.Generator().manual_seed(522)).to(DEV)
    sc = 1.0 / math.sqrt(D)
    args = [d[x] for x in ("q", "k", "v", "g", "beta")]
    full = kda.kda_chunk_bwd_varlen(*args, c["grad_out"].to(DEV), d["cu_seqlens"], sc,
                                    d["initial_state"], dsT)
    for cw in (1, 2):
        ws = kda.chunk_bwd_varlen_workspace(d["q"], d["v"], d["cu_seqlens"], window_chunks=cw)
        ws.fill_(0x33)
        got = kda.kda_chunk_bwd_varlen(*args, c["grad_out"].to(DEV), d["cu_seqlens"], sc,
                                       d["initial_state"], dsT, workspace=ws)
        torch.cuda.synchronize()
        for n, x, y in zip(NAMES, got, full):
            assert torch.equal(x, y), f"window {cw} {n}: windowed != one pass"


def test_windowed_backward_matches_oracle():
    from gated_delta_rule_102_amd import kda
    B, T, H, D = 1, 330, 2, 128
    d = kin.make_prefill(B, T, H, D, D, dtype=torch.bfloat16, seed=530, nonzero_state=True)
    c = kin.make_cotangents(B, T, H, D, D, dtype=torch.bfloat16, seed=531)
    g, gc = _dev(d), _dev(c)
    sc = 1.0 / math.sqrt(D)
    ws = kda.chunk_bwd_workspace(g["q"], g["v"], window_chunks=2)
    got = kda.kda_chunk_bwd(g["q"], g["k"], g["v"], g["g"], g["beta"], gc["grad_out"], sc,
                            g["initial_state"], gc["grad_final_state"], workspace=ws)
    torch.cuda.synchronize()
    ref = backward_oracle(d["q"], d["k"], d["v"], d["g"], d["beta"], sc, c["grad_out"],
                          d["initial_state"], c["grad_final_state"])
    for n, x in zip(NAMES, got):
        grad_close(n, x, ref[n], torch.bfloat16)
