"""GPU tests of prefill state snapshots (kda_chunk_fwd_snapshots, through the C ABI).

Snapshot i must be the state after min((i + 1) * S, T) tokens, i.e. the final
state the fp64 oracle computes on that prefix, within the same tolerances as any
final state; the last snapshot is the final state itself, and asking for
snapshots changes neither the outputs nor the final state.
"""
import math

import pytest
import torch

from gated_delta_rule_102_amd import inputs as kin
from tests.parity import assert_close, oracle_fixed, oracle_pair_slices

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


def _run(d, S):
    from gated_delta_rule_102_amd import kda
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    args = (g["q"], g["k"], g["v"], g["g"], g["beta"])
    out, fs, snaps = kda.kda_chunk_fwd_snapshots(*args, scale=d["scale"],
                                                 initial_state=g.get("initial_state"),
                                                 snapshot_tokens=S)
    out2, fs2 = kda.kda_chunk_fwd(*args, scale=d["scale"], initial_state=g.get("initial_state"))
    torch.cuda.synchronize()
    return out, fs, snaps, out2, fs2


def _prefix(d, t):
    return {k: (v[:, :t].contiguous() if isinstance(v, torch.Tensor) and k != "initial_state"
                else v) for k, v in d.items()}


@pytest.mark.parametrize("T,S,D,dtype", [(300, 128, 128, torch.bfloat16),
                                         (256, 64, 128, torch.bfloat16),
                                         (200, 512, 128, torch.bfloat16),
                                         (1100, 256, 64, torch.bfloat16),
                                         (190, 64, 64, torch.float32)])
def test_snapshots_match_oracle_on_prefixes(T, S, D, dtype):
    _check_snapshots(2, 3, T, S, D, dtype)


def test_snapshots_many_streams():
    """128 streams: snapshots from the two-kernel schedule's 64-column slices."""
    _check_snapshots(8, 16, 200, 64, 128, torch.bfloat16)


def test_snapshots_256_streams():
    """2 sequences x 128 heads (a plain call of this shape runs the fused kernel): a
    44-token tail after the last full interval."""
    _check_snapshots(2, 128, 300, 128, 128, torch.bfloat16)


def _check_snapshots(B, H, T, S, D, dtype):
    d = kin.make_prefill(B, T, H, D, D, dtype=dtype, seed=31 + T, nonzero_state=True)
    d["scale"] = 1.0 / math.sqrt(D)
    out, fs, snaps, out2, fs2 = _run(d, S)
    nsnap = -(-T // S)
    assert tuple(snaps.shape) == (B, H, nsnap, D, D)
    from gated_delta_rule_102_amd import kda
    if kda.prefill_schedule_name(B, T, H, D).startswith("fused"):
        # the plain call runs the fused kernel, the snapshot call the two-kernel
        # schedule: both against the oracle
        ref_o, ref_f = oracle_fixed(d)
        assert_close("output", out, ref_o.reshape(out.shape), dtype)
        assert_close("final state", fs, ref_f.reshape(fs.shape), dtype)
        assert_close("output (plain call)", out2, ref_o.reshape(out.shape), dtype)
    else:
        assert torch.equal(out, out2) and torch.equal(fs, fs2), "snapshots changed the results"
    assert torch.equal(snaps[:, :, -1], fs), "last snapshot differs from the final state"
    for i in range(nsnap):
        t = min((i + 1) * S, T)
        _, ref_s = oracle_fixed(_prefix(d, t))
        assert_close(f"snapshot {i} (t={t})", snaps[:, :, i], ref_s.reshape(B, H, D, D), dtype)


def test_snapshots_4x4096_full_size_sampled():
    """512-token snapshots of the 4 x 4096 x 16-head workload, on sampled pairs; the
    boundaries fall both inside and at the edges of the prefill's chunk windows."""
    w = kin.WORKLOADS["prefill_4x4096"]
    d = kin.make_workload(w)
    d["scale"] = w.scale_value()
    S = 512
    out, fs, snaps, out2, fs2 = _run(d, S)
    assert torch.equal(out, out2) and torch.equal(fs, fs2)
    pairs = [(0, 0), (1, 7), (3, 15)]
    for i in (0, 1, 3, 7):
        t = (i + 1) * S
        refs = oracle_pair_slices(d, pairs, [(n * w.T, t) for n in range(w.B)])
        got = torch.stack([snaps[n, h, i] for n, h in pairs])
        ref = torch.stack([torch.as_tensor(r[1]) for r in refs])
        assert_close(f"snapshot {i}", got, ref.numpy(), w.dtype)


def test_snapshot_interval_must_be_chunk_aligned():
    from gated_delta_rule_102_amd import kda
    d = kin.make_prefill(1, 128, 1, 128, 128, dtype=torch.bfloat16, seed=3, device=DEV)
    with pytest.raises(kda.KDAError) as e:
        kda.kda_chunk_fwd_snapshots(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                    snapshot_tokens=100)
    assert e.value.status == -2


def test_snapshots_across_windows():
    """T = 2100 spans three 16-chunk windows; snapshots every 512 tokens fall inside
    and at the edges of windows (the first window ends at token 1024)."""
    B, T, H, D, S = 1, 2100, 2, 128, 512
    d = kin.make_prefill(B, T, H, D, D, dtype=torch.bfloat16, seed=78, nonzero_state=True)
    d["scale"] = 1.0 / math.sqrt(D)
    out, fs, snaps, out2, fs2 = _run(d, S)
    assert torch.equal(out, out2) and torch.equal(fs, fs2)
    for i in range(-(-T // S)):
        t = min((i + 1) * S, T)
        _, ref_s = oracle_fixed(_prefix(d, t))
        assert_close(f"snapshot {i} (t={t})", snaps[:, :, i], ref_s.reshape(B, H, D, D), torch.bfloat16)


@pytest.mark.parametrize("lengths,H,S,D,dtype", [
    ([300, 0, 64, 1, 190, 700], 3, 128, 128, torch.bfloat16),
    ([130, 65, 256], 2, 64, 64, torch.float32),
    ([70 + 13 * i for i in range(48)], 3, 64, 128, torch.bfloat16),   # 144 streams
    ([300, 0, 64, 1, 190, 700, 129, 65, 256, 17, 1000, 3, 128, 511, 77, 640], 16, 128, 128,
     torch.bfloat16),                                                 # 256 streams
])
def test_varlen_snapshots_match_oracle(lengths, H, S, D, dtype):
    """kda_chunk_fwd_varlen_snapshots: every snapshot row of every sequence against the
    oracle's final state on that sequence's prefix; out and final state bitwise equal
    to kda_chunk_fwd_varlen (or, where that call runs the fused kernel, both against the
    oracle); each sequence's last row equal to its final state."""
    from gated_delta_rule_102_amd import kda
    d = kin.make_varlen(lengths, H, D, D, dtype=dtype, seed=71, nonzero_state=True)
    d["scale"] = 1.0 / math.sqrt(D)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    args = (g["q"], g["k"], g["v"], g["g"], g["beta"], g["cu_seqlens"])
    out, fs, snaps, rows = kda.kda_chunk_fwd_varlen_snapshots(
        *args, scale=d["scale"], initial_state=g["initial_state"], snapshot_tokens=S)
    out2, fs2 = kda.kda_chunk_fwd_varlen(*args, scale=d["scale"],
                                         initial_state=g["initial_state"])
    torch.cuda.synchronize()
    # a plain call that runs the fused kernel is checked against the oracle below
    fused = kda.prefill_schedule_name(len(lengths), max(lengths), H, D, dtype, varlen=True,
                                      total_T=sum(lengths)).startswith("fused")
    if not fused:
        assert torch.equal(out, out2) and torch.equal(fs, fs2), "snapshots changed the results"
    assert int(rows[-1]) == sum(-(-L // S) for L in lengths)
    assert tuple(snaps.shape) == (int(rows[-1]), H, D, D)
    cu = d["cu_seqlens"].tolist()
    checked = 0
    for n, L in enumerate(lengths):
        r0, r1 = int(rows[n]), int(rows[n + 1])
        assert r1 - r0 == -(-L // S)
        if L:
            assert torch.equal(snaps[r1 - 1], fs[n]), f"sequence {n}: last row != final state"
        # the oracle on every prefix of the small cases, on a few sequences of the large
        # ones (the longest among them)
        if len(lengths) > 8 and n not in (0, 5, 10, 13, 23, 47):
            continue
        if fused and L:
            sl = {x: d[x][:, cu[n]:cu[n] + L].contiguous() for x in ("q", "k", "v", "g", "beta")}
            sl["initial_state"] = d["initial_state"][n:n + 1]
            sl["scale"] = d["scale"]
            ref_o, ref_f = oracle_fixed(sl)
            for name, o in (("", out), (" (plain call)", out2)):
                assert_close(f"seq {n} output{name}", o[:, cu[n]:cu[n] + L],
                             ref_o.reshape(1, L, H, D), dtype)
            assert_close(f"seq {n} final state", fs[n], ref_f.reshape(H, D, D), dtype)
        for i in range(r1 - r0):
            t = min((i + 1) * S, L)
            sl = {x: d[x][:, cu[n]:cu[n] + t].contiguous() for x in ("q", "k", "v", "g", "beta")}
            sl["initial_state"] = d["initial_state"][n:n + 1]
            sl["scale"] = d["scale"]
            _, ref_s = oracle_fixed(sl)
            assert_close(f"seq {n} snapshot {i} (t={t})", snaps[r0 + i], ref_s.reshape(H, D, D),
                         dtype)
            checked += 1
    assert checked > 0
