"""kda_chunk_fwd_noalloc (scratch in a fixed per-GPU array, nothing allocated) against
kda_chunk_fwd and the fp64 oracle, through the C ABI: two calls in a row, the second
with a smaller input, so the second runs on what the first left in the array (the
segmented schedule's states, the windowed schedule's chunk operands); plus the fused
schedule (no scratch) and the refusal of sizes whose windows do not fit.
Tolerances of tests/parity.py."""
import ctypes
import math

import pytest
import torch

from gated_delta_rule_102_amd import inputs as kin
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


@pytest.mark.parametrize("first,second", [((4, 4096, 16), (2, 700, 16)),     # windows of 7
                                          ((1, 16400, 16), (1, 300, 24)),    # segmented, windowed
                                          ((2, 150, 128), (1, 300, 24))])    # fused, windowed
def test_noalloc_two_calls_match_kda_chunk_fwd(first, second):
    from gated_delta_rule_102_amd import kda
    for i, (B, T, H) in enumerate((first, second)):
        d = kin.make_prefill(B, T, H, 128, 128, seed=300 + i + B * T, nonzero_state=True)
        d["scale"] = 1.0 / math.sqrt(128)
        g = {x: d[x].to(DEV) for x in ("q", "k", "v", "g", "beta", "initial_state")}
        args = [g[x] for x in ("q", "k", "v", "g", "beta")]
        o, s = kda.kda_chunk_fwd_noalloc(*args, d["scale"], g["initial_state"])
        ro, rs = kda.kda_chunk_fwd(*args, d["scale"], g["initial_state"])
        torch.cuda.synchronize()
        print(f"call {i}: {B}x{T}x{H}, schedule of kda_chunk_fwd: "
              f"{kda.prefill_schedule_name(B, T, H, 128)}", flush=True)
        assert_close(f"noalloc {B}x{T}x{H} out vs kda_chunk_fwd", o, ro.float().cpu().numpy(),
                     torch.bfloat16)
        assert_close(f"noalloc {B}x{T}x{H} state vs kda_chunk_fwd", s, rs.cpu().numpy(),
                     torch.bfloat16)
        ref_o, ref_s = oracle_fixed(d)
        assert_close(f"noalloc {B}x{T}x{H} out vs oracle", o, ref_o.reshape(o.shape), torch.bfloat16)
        assert_close(f"noalloc {B}x{T}x{H} state vs oracle", s, ref_s.reshape(s.shape),
                     torch.bfloat16)


def test_noalloc_fp32_small_and_refusal():
    from gated_delta_rule_102_amd import kda
    d = kin.make_prefill(1, 256, 2, 64, 64, dtype=torch.float32, seed=1000)
    d["scale"] = 0.125
    g = {x: d[x].to(DEV) for x in ("q", "k", "v", "g", "beta")}
    o, s = kda.kda_chunk_fwd_noalloc(*(g[x] for x in ("q", "k", "v", "g", "beta")), 0.125)
    torch.cuda.synchronize()
    ref_o, ref_s = oracle_fixed(d)
    assert_close("noalloc fp32 out", o, ref_o.reshape(o.shape), torch.float32)
    assert_close("noalloc fp32 state", s, ref_s.reshape(s.shape), torch.float32)
    # fp32, d = 64, 1000 tokens (16 chunks), 400 heads: the carried states plus two
    # one-chunk windows exceed 64 MiB; refused before anything is enqueued (the buffer
    # is sized for the call all the same)
    lib = kda.load_library()
    x = torch.zeros(1 * 1000 * 400 * 64, dtype=torch.float32, device=DEV)
    p = ctypes.c_void_p(x.data_ptr())
    rc = lib.kda_chunk_fwd_noalloc(p, p, p, p, p, None, p, None, 1, 1000, 400, 64, 64, 0.1, 1,
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == -8
