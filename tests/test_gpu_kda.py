"""GPU parity tests: libkda.so (through its C ABI) against the fp64 CPU oracle.

Every case feeds bit-identical seeded inputs to both sides and compares outputs
and final states element by element with the tolerances in tests/parity.py.
Cases here span several 64-token chunks and ragged tails; the four full-size
workloads are compared in full in test_gpu_full_size.py.
"""
import math

import numpy as np
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


def _to(d, device):
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def _run_prefill(d):
    from gated_delta_rule_102_amd import kda
    g = _to(d, DEV)
    out, fs = kda.kda_chunk_fwd(g["q"], g["k"], g["v"], g["g"], g["beta"], scale=d["scale"],
                                initial_state=g.get("initial_state"))
    torch.cuda.synchronize()
    return out, fs


def _compare_fixed(d, tag):
    out, fs = _run_prefill(d)
    ref_out, ref_s = oracle_fixed(d)
    B, T, H, dv = out.shape
    assert_close(f"{tag} out", out, ref_out.reshape(B, T, H, dv), d["q"].dtype)
    assert_close(f"{tag} state", fs, ref_s.reshape(fs.shape), d["q"].dtype)


# ------------------------------------------------------------------ decode


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_steps_match_oracle(D, dtype):
    from gated_delta_rule_102_amd import kda
    steps, B, H = 8, 5, 3
    d = kin.make_decode(steps, B, H, D, D, dtype=dtype, seed=11)
    scale = 1.0 / math.sqrt(D)
    state = d["state"].to(DEV).clone()
    outs = []
    for s in range(steps):
        outs.append(kda.kda_decode_step(d["q"][s].to(DEV), d["k"][s].to(DEV), d["v"][s].to(DEV),
                                        d["g"][s].to(DEV), d["beta"][s].to(DEV), state,
                                        scale=scale))
    torch.cuda.synchronize()
    out = torch.stack(outs)                                     # [steps, B, H, D]
    # the oracle sees the same tokens as B sequences of `steps` tokens
    seq = {x: d[x].transpose(0, 1).contiguous() for x in ("q", "k", "v", "g")}
    seq["beta"] = d["beta"].transpose(0, 1).contiguous()
    ref_out, ref_s = oracle_fixed({**seq, "initial_state": d["state"], "scale": scale})
    assert_close("decode out", out.transpose(0, 1), ref_out.reshape(B, steps, H, D), dtype)
    assert_close("decode state", state, ref_s.reshape(B, H, D, D), dtype)


# ------------------------------------------------------------------ prefill


def test_prefill_fp32_small_workload():
    """fp32, B=1, H=2, T=256, d=64, scale 1/8, zero initial state: rel-L2 <= 1e-4."""
    d = kin.make_workload(kin.WORKLOADS["fp32_small"])
    _compare_fixed(d, "fp32_small")


@pytest.mark.parametrize("T", [1, 17, 63, 64, 65, 127, 200])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_bf16_ragged(T, D):
    d = kin.make_prefill(2, T, 3, D, D, dtype=torch.bfloat16, seed=100 + T, nonzero_state=True)
    d["scale"] = 1.0 / math.sqrt(D)
    _compare_fixed(d, f"bf16 T={T} D={D}")


@pytest.mark.parametrize("T", [1, 63, 130])
def test_prefill_fp32_ragged(T):
    d = kin.make_prefill(2, T, 2, 64, 64, dtype=torch.float32, seed=200 + T, nonzero_state=True)
    d["scale"] = 0.125
    _compare_fixed(d, f"fp32 T={T}")


@pytest.mark.parametrize("B,T,H,D,dtype", [(2, 1100, 16, 128, torch.bfloat16),
                                           (1, 1100, 40, 64, torch.bfloat16),
                                           (2, 1100, 16, 64, torch.float32)])
def test_prefill_windows_32_streams(B, T, H, D, dtype):
    """32 to 127 streams over two windows (the second ragged): the windowed schedule
    with 32-column scan slices, both head sizes and dtypes."""
    d = kin.make_prefill(B, T, H, D, D, dtype=dtype, seed=400 + H, nonzero_state=True)
    d["scale"] = 1.0 / math.sqrt(D)
    _compare_fixed(d, f"{B}x{T}x{H} D={D} {dtype}")


@pytest.mark.parametrize("B,T,H,D,dtype", [(8, 200, 16, 128, torch.bfloat16),
                                           (4, 65, 40, 128, torch.bfloat16),
                                           (8, 130, 16, 64, torch.float32)])
def test_prefill_many_streams(B, T, H, D, dtype):
    """128 and more (sequence, head) streams: the two-kernel schedule with 64-column
    scan slices (whole states at d = 64), ragged tails, nonzero initial state."""
    d = kin.make_prefill(B, T, H, D, D, dtype=dtype, seed=300 + T, nonzero_state=True)
    d["scale"] = 1.0 / math.sqrt(D)
    _compare_fixed(d, f"{B}x{T}x{H} D={D} {dtype}")


@pytest.mark.parametrize("mode", ["floor", "slow"])
def test_prefill_decay_extremes(mode):
    """g = -5 everywhere (the bound: sub-tile factors reach e^80) and g in
    [-0.05, 0] (almost no forgetting)."""
    d = kin.make_prefill(1, 300, 4, 128, 128, dtype=torch.bfloat16, seed=7, nonzero_state=True)
    if mode == "floor":
        d["g"] = torch.full_like(d["g"], -5.0)
    else:
        d["g"] = (-0.05 * torch.rand(d["g"].shape, generator=torch.Generator().manual_seed(3))
                  ).to(torch.bfloat16)
    d["scale"] = 1.0 / math.sqrt(128)
    _compare_fixed(d, f"decay {mode}")


# ------------------------------------------------------------------ varlen


def _run_varlen(d):
    from gated_delta_rule_102_amd import kda
    g = _to(d, DEV)
    out, fs = kda.kda_chunk_fwd_varlen(g["q"], g["k"], g["v"], g["g"], g["beta"],
                                       g["cu_seqlens"], scale=d["scale"],
                                       initial_state=g.get("initial_state"))
    torch.cuda.synchronize()
    return out, fs


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.bfloat16, 64),
                                     (torch.float32, 64)])
def test_varlen_matches_oracle(dtype, D):
    lengths = [5, 0, 130, 64, 1, 200, 63]
    d = kin.make_varlen(lengths, 3, D, D, dtype=dtype, seed=31, nonzero_state=True,
                        split_decay=True)
    d["scale"] = 1.0 / math.sqrt(D)
    out, fs = _run_varlen(d)
    from oracle import oracle_forward
    ref_out, ref_s = oracle_forward(d["q"][0], d["k"][0], d["v"][0], d["g"][0], d["beta"][0],
                                    d["scale"], cu_seqlens=d["cu_seqlens"].numpy(),
                                    initial_state=d["initial_state"])
    assert_close("varlen out", out[0], ref_out, dtype)
    assert_close("varlen state", fs, ref_s.reshape(fs.shape), dtype)


# ------------------------------------------------------------------ invariants


def test_split_sequence_state_passing_gpu():
    from gated_delta_rule_102_amd import kda
    d = _to(kin.make_prefill(2, 300, 4, 128, 128, seed=41, nonzero_state=True), DEV)
    sc = 1.0 / math.sqrt(128)
    out, fs = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], sc, d["initial_state"])
    cut = 100
    a = {x: d[x][:, :cut].contiguous() for x in ("q", "k", "v", "g", "beta")}
    b = {x: d[x][:, cut:].contiguous() for x in ("q", "k", "v", "g", "beta")}
    oa, sa = kda.kda_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], sc, d["initial_state"])
    ob, sb = kda.kda_chunk_fwd(b["q"], b["k"], b["v"], b["g"], b["beta"], sc, sa)
    torch.cuda.synchronize()
    ref_o, ref_s = oracle_fixed({**{x: d[x].cpu() for x in ("q", "k", "v", "g", "beta")},
                                 "initial_state": d["initial_state"].cpu(), "scale": sc})
    assert_close("split out", torch.cat([oa, ob], 1), ref_o.reshape(out.shape), torch.bfloat16)
    assert_close("split state", sb, ref_s.reshape(fs.shape), torch.bfloat16)
    assert_close("split vs whole", torch.cat([oa, ob], 1), out.float().cpu().numpy(), torch.bfloat16)


def test_decode_equals_prefill():
    """64 decode steps from S0 agree with one prefill of those 64 tokens."""
    from gated_delta_rule_102_amd import kda
    d = kin.make_decode(64, 3, 2, 128, 128, seed=43)
    sc = 1.0 / math.sqrt(128)
    dd = _to(d, DEV)
    state = dd["state"].clone()
    outs = [kda.kda_decode_step(dd["q"][s], dd["k"][s], dd["v"][s], dd["g"][s], dd["beta"][s],
                                state, scale=sc) for s in range(64)]
    seq = {x: dd[x].transpose(0, 1).contiguous() for x in ("q", "k", "v", "g", "beta")}
    out, fs = kda.kda_chunk_fwd(seq["q"], seq["k"], seq["v"], seq["g"], seq["beta"], sc,
                                dd["state"])
    torch.cuda.synchronize()
    assert_close("decode vs prefill out", torch.stack(outs, 1), out.float().cpu().numpy(),
                 torch.bfloat16)
    assert_close("decode vs prefill state", state, fs.cpu().numpy(), torch.bfloat16)


def test_varlen_equals_separate_calls_and_is_deterministic():
    from gated_delta_rule_102_amd import kda
    lengths = [70, 3, 129]
    d = kin.make_varlen(lengths, 2, 128, 128, seed=47, nonzero_state=True)
    d["scale"] = 1.0 / math.sqrt(128)
    out, fs = _run_varlen(d)
    out2, fs2 = _run_varlen(d)
    assert torch.equal(out, out2) and torch.equal(fs, fs2), "run-to-run results differ"
    cu = d["cu_seqlens"].tolist()
    g = _to(d, DEV)
    for n, L in enumerate(lengths):
        sl = slice(cu[n], cu[n + 1])
        o, s = kda.kda_chunk_fwd(*(g[x][:, sl].contiguous() for x in ("q", "k", "v", "g", "beta")),
                                 d["scale"], g["initial_state"][n:n + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(o[0], out[0, sl]), f"sequence {n} output differs from its own call"
        assert torch.equal(s[0], fs[n]), f"sequence {n} state differs from its own call"


def test_in_place_state():
    from gated_delta_rule_102_amd import kda
    d = _to(kin.make_prefill(2, 150, 3, 128, 128, seed=53, nonzero_state=True), DEV)
    sc = 1.0 / math.sqrt(128)
    out, fs = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], sc, d["initial_state"])
    st = d["initial_state"].clone()
    out2, fs2 = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], sc, st,
                                  final_state=st)
    torch.cuda.synchronize()
    assert fs2.data_ptr() == st.data_ptr()
    assert torch.equal(out, out2) and torch.equal(fs, st)


def test_no_final_state_and_zero_initial():
    from gated_delta_rule_102_amd import kda
    d = _to(kin.make_prefill(1, 70, 2, 64, 64, seed=59), DEV)
    out, fs = kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], 0.125,
                                output_final_state=False)
    torch.cuda.synchronize()
    assert fs is None
    ref_o, _ = oracle_fixed({**{x: d[x].cpu() for x in ("q", "k", "v", "g", "beta")},
                             "scale": 0.125})
    assert_close("no-final out", out, ref_o.reshape(out.shape), torch.bfloat16)


# ------------------------------------------------------------------ ABI errors


def test_abi_error_codes_launch_nothing():
    import ctypes
    from gated_delta_rule_102_amd import kda
    lib = kda.load_library()
    x = torch.zeros(2 * 64 * 2 * 128, dtype=torch.bfloat16, device=DEV)
    o = torch.full((2 * 64 * 2 * 128,), 7.0, dtype=torch.bfloat16, device=DEV)
    p = ctypes.c_void_p(x.data_ptr())
    po = ctypes.c_void_p(o.data_ptr())
    mis = ctypes.c_void_p(x.data_ptr() + 2)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    f = lib.kda_chunk_fwd
    assert f(None, p, p, p, p, None, po, None, 2, 64, 2, 128, 128, 0.1, 0, s) == -1
    assert f(p, p, p, p, p, None, po, None, 0, 64, 2, 128, 128, 0.1, 0, s) == -2
    assert f(p, p, p, p, p, None, po, None, 2, 64, 2, 96, 96, 0.1, 0, s) == -3
    assert f(p, p, p, p, p, None, po, None, 2, 64, 2, 128, 64, 0.1, 0, s) == -3
    assert f(p, p, p, p, p, None, po, None, 2, 64, 2, 64, 128, 0.1, 1, s) == -3
    assert f(p, p, p, p, p, None, po, None, 2, 64, 2, 128, 128, 0.1, 5, s) == -4
    assert f(mis, p, p, p, p, None, po, None, 2, 64, 2, 128, 128, 0.1, 0, s) == -5
    assert lib.kda_decode_step(p, p, p, p, p, None, po, 2, 2, 128, 128, 0.1, 0, s) == -1
    assert lib.kda_chunk_fwd_varlen(p, p, p, p, p, None, po, None, None, 2, 64, 2, 128, 128,
                                    0.1, 0, s) == -1
    torch.cuda.synchronize()
    assert torch.all(o == 7.0), "a rejected call wrote its output"
    assert kda.kda_status_string(-3).startswith("dk and dv")


def test_prefill_several_windows_small():
    """Fixed-length prefill longer than one 16-chunk window (T = 2100: three
    windows, the last one ragged) with a nonzero state, element by element against
    the oracle: exercises the state carried between windows."""
    d = kin.make_prefill(2, 2100, 2, 128, 128, dtype=torch.bfloat16, seed=77, nonzero_state=True)
    d["scale"] = 1.0 / math.sqrt(128)
    _compare_fixed(d, "3 windows")


# ------------------------------------------------------------ caller workspace


@pytest.mark.parametrize("B,T,H,D,dtype", [(2, 150, 3, 128, torch.bfloat16),
                                           (1, 2100, 4, 128, torch.bfloat16),
                                           (4, 4096, 16, 128, torch.bfloat16),
                                           (1, 300, 2, 64, torch.float32)])
def test_workspace_entry_point_equals_self_allocating(B, T, H, D, dtype):
    """kda_chunk_fwd_ws on a caller workspace runs the same kernels as kda_chunk_fwd:
    bitwise-equal outputs and states (one window, several windows with a ragged last
    one, the bench workload, fp32), also when the workspace held garbage and when
    two calls reuse it back to back; the first call is also checked against the
    oracle on the small cases."""
    from gated_delta_rule_102_amd import kda
    d = kin.make_prefill(B, T, H, D, D, dtype=dtype, seed=31 + T, nonzero_state=True)
    d["scale"] = 1.0 / math.sqrt(D)
    g = _to(d, DEV)
    args = (g["q"], g["k"], g["v"], g["g"], g["beta"])
    ref_out, ref_fs = kda.kda_chunk_fwd(*args, scale=d["scale"], initial_state=g["initial_state"])
    ws = kda.chunk_fwd_workspace(g["q"], g["v"])
    ws.fill_(0xA5)
    for rep in range(2):
        out, fs = kda.kda_chunk_fwd(*args, scale=d["scale"], initial_state=g["initial_state"],
                                    workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"rep {rep}: out differs from kda_chunk_fwd"
        assert torch.equal(fs, ref_fs), f"rep {rep}: final state differs from kda_chunk_fwd"
    if B * T * H <= 4 * 2100:
        o_ref, s_ref = oracle_fixed(d)
        assert_close("ws out", out, o_ref.reshape(out.shape), dtype)
        assert_close("ws state", fs, s_ref.reshape(fs.shape), dtype)


def test_workspace_too_small_is_rejected():
    from gated_delta_rule_102_amd import kda
    d = kin.make_prefill(1, 128, 2, 128, 128, dtype=torch.bfloat16, seed=3)
    g = _to(d, DEV)
    need = kda.kda_chunk_fwd_workspace_size(1, 128, 2, 128, 128, torch.bfloat16)
    assert need > 0
    small = torch.empty(need // 2, dtype=torch.uint8, device=DEV)
    with pytest.raises(kda.KDAError) as e:
        kda.kda_chunk_fwd(g["q"], g["k"], g["v"], g["g"], g["beta"], workspace=small)
    assert e.value.status == -8


def test_workspace_blocks_across_streams():
    """Self-allocating calls reuse the library's workspace blocks: calls on two
    streams, interleaved, a larger call after smaller ones (the free blocks that are
    too small go back to the pool), and smaller ones again; every result is bitwise
    equal to the same call run alone on the default stream."""
    from gated_delta_rule_102_amd import kda
    shapes = [(2, 300, 4), (1, 1100, 8), (4, 640, 16), (2, 130, 2)]
    data = []
    for i, (B, T, H) in enumerate(shapes):
        d = kin.make_prefill(B, T, H, 128, 128, dtype=torch.bfloat16, seed=90 + i,
                             nonzero_state=True)
        data.append(_to(d, DEV))

    def call(g):
        return kda.kda_chunk_fwd(g["q"], g["k"], g["v"], g["g"], g["beta"],
                                 initial_state=g["initial_state"])

    refs = []
    for g in data:
        o, s = call(g)
        torch.cuda.synchronize()
        refs.append((o.clone(), s.clone()))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    results = []
    for rep in range(3):
        for i, g in enumerate(data):
            with torch.cuda.stream(streams[(i + rep) % 2]):
                o, s = call(g)
                results.append((i, o, s))
    torch.cuda.synchronize()
    for i, o, s in results:
        assert torch.equal(o, refs[i][0]) and torch.equal(s, refs[i][1]), f"call {i} differs"


def test_prefill_seeded_random_shapes():
    """Twelve seeded random shapes (batch, length, heads, head size, dtype, initial
    state present or not) through kda_chunk_fwd, each against the oracle: lengths
    1..2300 hit one or several windows with ragged tails, stream counts 1..160 hit
    every scan slice width and both schedules."""
    rng = np.random.default_rng(20261203)
    for case in range(12):
        dtype = torch.float32 if rng.random() < 0.25 else torch.bfloat16
        D = 64 if dtype == torch.float32 else int(rng.choice([64, 128]))
        B = int(rng.integers(1, 9))
        H = int(rng.integers(1, 21))
        T = int(rng.integers(1, 2301)) if B * H <= 16 else int(rng.integers(1, 400))
        d = kin.make_prefill(B, T, H, D, D, dtype=dtype, seed=500 + case,
                             nonzero_state=bool(rng.random() < 0.7))
        d["scale"] = 1.0 / math.sqrt(D)
        print(f"case {case}: B={B} T={T} H={H} D={D} {dtype}", flush=True)
        _compare_fixed(d, f"random case {case} (B={B} T={T} H={H} D={D} {dtype})")
