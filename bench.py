"""Benchmark: KDA chunked prefill (and decode) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one kda_chunk_fwd call over the prefill workload B=4, H=16, T=4096,
dk=dv=128, bf16 q/k/v/g/beta, fp32 initial and final states (every prefill row
of the hot path: decay factors, intra-chunk products, UT transform, inter-chunk
state propagation, state in/out).  W untimed steps, then K timed steps between
two device synchronisations; inputs are resident in HBM before timing starts
and two input sets alternate so consecutive steps do not reuse cached inputs.
The decode row (single-token update of 256 x 32 fp32 states, d=128, 64
consecutive kda_decode_step calls) is timed in the same run and reported in the
"decode" object.  Kernel durations come from HIP events recorded on the stream
the library launches on; "roofline" relates the prefill kernel's algorithmic
HBM bytes to its average duration.  The "prologue" object times the same prefill
from raw activations through kda_chunk_fwd_prologue (gate and normalisation
fused into the kernels' loads).  The "backward" object times kda_chunk_bwd (all
gradients of the same prefill) and relates its dense matrix work to the bf16 and
fp32 matrix peaks.  "snapshots" times the same prefill keeping the state every
1024 tokens (kda_chunk_fwd_snapshots).  "context" times each step of the
context-parallel schedule (segment prefill, kda_chunk_transition,
kda_state_compose) at B=1, T=65536, H=32 in 8 segments, and the whole schedule
on one GPU.  "varlen" times kda_chunk_fwd_varlen on 64 packed sequences of
log-uniform lengths in [1024, 65536] (32 heads).  "cpu_baseline" times the fp64 CPU oracle on a bounded sample of the
same workload.  One JSON line is printed.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published
FP32_MFMA_PEAK_TFLOPS = 157.3   # MI355X dense fp32 matrix, published
CHUNK = 64
METRIC = "KDA prefill tokens/s + % bf16 MFMA peak; decode state GB/s + % HBM peak"


def prefill_bytes(B, T, H, d, elt, state_in=True, state_out=True):
    """Algorithmic HBM bytes of one prefill: q, k, g, v, beta read once, out written
    once, states read/written once (per token-head (3d + 2d + 1) * elt)."""
    tok = B * T * H * (5 * d + 1) * elt
    st = B * H * d * d * 4 * (int(state_in) + int(state_out))
    return tok + st


def prefill_flops(B, T, H, d):
    """Triangle-aware flops of the chunked algorithm as implemented, per token-head:
    Cd (key Gram) + Cd (query-key) + 4d^2 ([Q;K] S) + Cd (T X) + Cd (M Delta)
    + 2d^2 (K^T Delta) + C^2/3 (triangular inverse) = 4Cd + 6d^2 + C^2/3; the
    full-rectangle count doubles the four triangular products: 8Cd + 6d^2 + C^2/3."""
    C = CHUNK
    tri = 4 * C * d + 6 * d * d + C * C / 3
    full = 8 * C * d + 6 * d * d + C * C / 3
    n = B * T * H
    return n * tri, n * full


PREFILL_SRC = os.path.join(ROOT, "gated_delta_rule_102_amd", "csrc", "kda_prefill.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_4x4096_hbm_traffic.txt")


def source_digest(path=PREFILL_SRC):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per prefill call from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, scaled by the plain-copy calibration; None if that summary was taken
    on a different version of the prefill kernels."""
    try:
        vals = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    key, val = line.split(":", 1)
                    vals[key.strip()] = val.strip()
        if vals.get("kernel_source_sha256") != source_digest():
            return None
        return float(vals["hbm_bytes_per_call"])
    except (OSError, KeyError, ValueError):
        return None


def pmc_copy(torch, nbytes=256 << 20, reps=3):
    """A plain device copy of known size, for scaling the PMC byte counters."""
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_copy_bytes_read": nbytes, "pmc_copy_bytes_written": nbytes,
                      "reps": reps}))


def backward_flops(B, T, H, d):
    """Dense matrix-product flops of the backward per 64-token chunk and head, summed
    over its four kernels at d = 128 and counted in 16x16x4 products (2048 flops
    each): operand prep 1984, forward state scan 2560, reverse scan 4096, and in the
    per-chunk gradient kernel operand gradients 4096, 64x64 algebra 3072 and
    decayed products 1280 (dense tiles, including the zero upper triangles of the
    triangular factors).  For bf16 inputs most of them run as bf16 16x16x32
    products (8 of these each)."""
    assert d == 128
    per_chunk = (1984 + 2560 + 4096 + 4096 + 3072 + 1280) * 2048
    return B * H * (-(-T // CHUNK)) * per_chunk


def decode_bytes(B, H, d, elt):
    """Per step: the fp32 state read and written once, plus the token's inputs/output."""
    state = B * H * d * d * 4 * 2
    return state, state + B * H * (5 * d + 1) * elt


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-reps", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-prologue", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-snapshots", action="store_true")
    ap.add_argument("--no-context", action="store_true")
    ap.add_argument("--no-varlen", action="store_true")
    ap.add_argument("--pmc-copy", action="store_true",
                    help="only run a plain 256 MiB copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the KDA path here has no multi-GPU mode "
              "(sequences and heads shard across GPUs with no communication). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from gated_delta_rule_102_amd import inputs as kin
    from gated_delta_rule_102_amd import kda

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.pmc_copy:
        pmc_copy(torch)
        return
    kda.load_library()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    w = kin.WORKLOADS["prefill_4x4096"]
    B, T, H, d = w.B, w.T, w.H, w.dk
    sets = [kin.make_workload(w, device=dev, seed=w.seed + i) for i in range(2)]
    outs = [torch.empty((B, T, H, d), dtype=w.dtype, device=dev) for _ in sets]
    finals = [torch.empty((B, H, d, d), dtype=torch.float32, device=dev) for _ in sets]
    scale = w.scale_value()
    stream = torch.cuda.current_stream()

    # one workspace, allocated before timing and reused by every call on this stream
    # (kda_chunk_fwd_ws): the call then allocates and frees nothing
    wsbuf = kda.chunk_fwd_workspace(sets[0]["q"], sets[0]["v"])

    def step(i, workspace=wsbuf):
        s = sets[i % 2]
        kda.kda_chunk_fwd(s["q"], s["k"], s["v"], s["g"], s["beta"], scale,
                          s["initial_state"], out=outs[i % 2], final_state=finals[i % 2],
                          workspace=workspace)

    # the same calls through the self-allocating entry point (kda_chunk_fwd), timed
    # first, for context
    for i in range(args.warmup):
        step(i, None)
    torch.cuda.synchronize()
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t1 = time.perf_counter()
    ea.record(stream)
    for i in range(args.steps):
        step(i, None)
    eb.record(stream)
    torch.cuda.synchronize()
    self_alloc_wall = (time.perf_counter() - t1) / args.steps
    self_alloc_ms = ea.elapsed_time(eb) / args.steps

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # one HIP event pair on the launch stream around the K timed steps: per-step
    # events would put their own host cost between the calls
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_avg_s = ev0.elapsed_time(ev1) / args.steps / 1e3

    tokens = B * T
    value = tokens * args.steps / wall
    nbytes = prefill_bytes(B, T, H, d, 2)
    fl_tri, fl_full = prefill_flops(B, T, H, d)
    achieved_gbs = nbytes / kern_avg_s / 1e9
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill_4x4096", "B": B, "T": T, "H": H, "dk": d, "dv": d,
                   "chunk": CHUNK, "state": "fp32, initial ~0.1 N(0,1), final returned",
                   "global_batch": B, "seq_len": T, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved_gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic(),
                     "kernel": "kda_chunk_fwd_ws = chunk_prep8_kernel (chunk operands, 8 "
                               "wavefronts per (chunk, head)) + state_scan_kernel<128,32,bf16> "
                               "(serial state scan, 32-column slices); time per call from one "
                               "HIP event pair around the timed steps",
                     "kernel_ms": kern_avg_s * 1e3, "algorithmic_bytes": nbytes,
                     "kernel_source_sha256": source_digest()},
        "prefill": {
            "entry_point": "kda_chunk_fwd_ws (caller workspace, "
                           f"{wsbuf.numel() / 2**20:.0f} MiB)",
            "kernel_ms_avg": kern_avg_s * 1e3,
            "self_allocating_kda_chunk_fwd": {
                "ms_per_call_events": self_alloc_ms, "ms_per_call_wall": self_alloc_wall * 1e3,
                "note": "timed before the caller-workspace steps; workspace from the blocks "
                        "the library keeps per device (taken after an event wait, released "
                        "with an event record; nothing allocated or freed once warm)"},
            "token_heads_per_s": tokens * H / kern_avg_s,
            "tflops_tri": fl_tri / kern_avg_s / 1e12, "tflops_full": fl_full / kern_avg_s / 1e12,
            "mfma_frac_tri": fl_tri / kern_avg_s / 1e12 / BF16_MFMA_PEAK_TFLOPS,
            "mfma_frac_full": fl_full / kern_avg_s / 1e12 / BF16_MFMA_PEAK_TFLOPS,
            "flop_convention": "tri = 4Cd + 6d^2 + C^2/3 per token-head (C=64); "
                               "full = 8Cd + 6d^2 + C^2/3",
        },
    }
    del sets, outs, finals, wsbuf
    torch.cuda.empty_cache()

    if not args.no_prologue:
        # the same prefill from raw activations, with the gate/normalisation prologue
        # fused into the kernels' loads (kda_chunk_fwd_prologue): same bytes moved
        raw = [kin.make_prefill_raw(B, T, H, d, d, dtype=w.dtype, seed=w.seed + 10 + i,
                                    device=dev, nonzero_state=True) for i in range(2)]
        pout = torch.empty((B, T, H, d), dtype=w.dtype, device=dev)
        pfin = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)

        def pstep(i):
            r = raw[i % 2]
            kda.kda_chunk_fwd_prologue(r["q_raw"], r["k_raw"], r["v"], r["g_raw"], r["beta_raw"],
                                       scale, r["initial_state"], out=pout, final_state=pfin)

        for i in range(args.warmup):
            pstep(i)
        torch.cuda.synchronize()
        pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for i in range(args.steps):
            pev[i][0].record(stream)
            pstep(i)
            pev[i][1].record(stream)
        torch.cuda.synchronize()
        p_s = sum(a.elapsed_time(b) for a, b in pev) / len(pev) / 1e3
        result["prologue"] = {
            "entry_point": "kda_chunk_fwd_prologue", "workload": "prefill_4x4096 (raw activations)",
            "kernel_ms_avg": p_s * 1e3, "tokens_per_s": B * T / p_s,
            "achieved_GBps": nbytes / p_s / 1e9, "hbm_frac": nbytes / p_s / 1e9 / HBM_PEAK_GBS,
        }
        del raw, pout, pfin
        torch.cuda.empty_cache()

    def event_ms(fn, n):
        """Mean duration of fn() on the stream over n calls after one warm-up call."""
        fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / n

    if not args.no_snapshots:
        # the same prefill keeping the state every 1024 tokens (prefix-cache snapshots)
        sset = kin.make_workload(w, device=dev)
        snap_tokens = 1024
        sms = event_ms(lambda: kda.kda_chunk_fwd_snapshots(
            sset["q"], sset["k"], sset["v"], sset["g"], sset["beta"], scale,
            sset["initial_state"], snapshot_tokens=snap_tokens), max(3, min(args.steps, 10)))
        result["snapshots"] = {
            "entry_point": "kda_chunk_fwd_snapshots", "workload": "prefill_4x4096",
            "snapshot_tokens": snap_tokens, "snapshots_per_sequence": -(-T // snap_tokens),
            "call_ms_avg": sms, "tokens_per_s": B * T / (sms / 1e3),
            "vs_plain_prefill": sms / (kern_avg_s * 1e3),
        }
        del sset
        torch.cuda.empty_cache()

    if not args.no_backward:
        # all gradients of the same prefill (kda_chunk_bwd): forward recomputed
        # inside; bf16 matrix-core operands with fp32 accumulation for bf16 inputs
        bset = kin.make_workload(w, device=dev)
        cot = kin.make_cotangents(B, T, H, d, d, dtype=w.dtype, seed=w.seed + 20, device=dev)

        def bstep():
            return kda.kda_chunk_bwd(bset["q"], bset["k"], bset["v"], bset["g"], bset["beta"],
                                     cot["grad_out"], scale, bset["initial_state"],
                                     cot["grad_final_state"])

        for _ in range(2):
            bstep()
        torch.cuda.synchronize()
        nb = max(3, min(args.steps, 10))
        bev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(nb)]
        for i in range(nb):
            bev[i][0].record(stream)
            grads = bstep()
            bev[i][1].record(stream)
            del grads
        torch.cuda.synchronize()
        b_s = sum(a.elapsed_time(b) for a, b in bev) / nb / 1e3
        bfl = backward_flops(B, T, H, d)
        result["backward"] = {
            "entry_point": "kda_chunk_bwd", "workload": "prefill_4x4096 gradients",
            "calls": nb, "call_ms_avg": b_s * 1e3, "tokens_per_s": B * T / b_s,
            "matrix_tflops": bfl / b_s / 1e12,
            "frac_of_bf16_mfma_peak": bfl / b_s / 1e12 / BF16_MFMA_PEAK_TFLOPS,
            "frac_of_fp32_mfma_peak": bfl / b_s / 1e12 / FP32_MFMA_PEAK_TFLOPS,
            "flop_convention": "dense matrix products, 35.0 MFLOP per chunk and head (17088 "
                               "16x16x4 equivalents); bf16 operands with fp32 accumulation for "
                               "the products over 32 or more terms, fp32 for the rest",
        }
        del bset, cot
        torch.cuda.empty_cache()

    if not args.no_varlen:
        # packed variable-length prefill: 64 sequences, log-uniform lengths in
        # [1024, 65536], 32 heads, half at g = -5 (kda_chunk_fwd_varlen)
        wv = kin.WORKLOADS["varlen_64seq"]
        dvl = kin.make_workload(wv, device=dev)
        vargs = [dvl[x] for x in ("q", "k", "v", "g", "beta")]
        vscale = wv.scale_value()
        total = int(dvl["cu_seqlens"][-1])
        for _ in range(2):
            kda.kda_chunk_fwd_varlen(*vargs, dvl["cu_seqlens"], vscale)
        torch.cuda.synchronize()
        nv = 3
        va, vb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        va.record(stream)
        for _ in range(nv):
            kda.kda_chunk_fwd_varlen(*vargs, dvl["cu_seqlens"], vscale)
        vb.record(stream)
        torch.cuda.synchronize()
        v_s = va.elapsed_time(vb) / nv / 1e3
        vbytes = total * wv.H * (5 * wv.dk + 1) * 2 + 64 * wv.H * wv.dk * wv.dv * 4
        result["varlen"] = {
            "entry_point": "kda_chunk_fwd_varlen", "workload": "varlen_64seq",
            "sequences": 64, "tokens": total, "H": wv.H, "d": wv.dk, "calls": nv,
            "call_ms_avg": v_s * 1e3, "tokens_per_s": total / v_s,
            "achieved_GBps": vbytes / v_s / 1e9, "hbm_frac": vbytes / v_s / 1e9 / HBM_PEAK_GBS,
        }
        del dvl, vargs
        torch.cuda.empty_cache()

    if not args.no_context:
        # context parallelism on one GPU, prefill_1x65536 in 8 segments of 8192 tokens:
        # every step of the schedule, and the path one rank of eight would take
        wc = kin.WORKLOADS["prefill_1x65536"]
        cset = kin.make_workload(wc, device=dev)
        Tc, nseg = cset["q"].shape[1], 8
        seg = Tc // nseg
        cq, ck, cv, cg, cb = (cset[x] for x in ("q", "k", "v", "g", "beta"))
        sq, sk, sv, sg, sb = (x[:, :seg].contiguous() for x in (cq, ck, cv, cg, cb))
        cscale = wc.scale_value()
        single = event_ms(lambda: kda.kda_chunk_fwd(cq, ck, cv, cg, cb, cscale), 3)
        seg_fwd = event_ms(lambda: kda.kda_chunk_fwd(sq, sk, sv, sg, sb, cscale), 5)
        seg_tr = event_ms(lambda: kda.kda_chunk_transition(sq, sk, sg, sb), 5)
        Pm = torch.randn((nseg, 1, wc.H, wc.dk, wc.dk), device=dev) * 0.01
        Rm = torch.randn((nseg, 1, wc.H, wc.dk, wc.dv), device=dev)
        comp = event_ms(lambda: kda.kda_state_compose(Pm, Rm), 5)
        serial = event_ms(lambda: kda.chunk_fwd_context_parallel(cq, ck, cv, cg, cb, seg, cscale), 2)
        result["context"] = {
            "entry_points": "kda_chunk_transition, kda_state_compose (with kda_chunk_fwd)",
            "workload": "prefill_1x65536 in 8 segments of 8192 tokens",
            "single_pass_prefill_ms": single, "segment_prefill_ms": seg_fwd,
            "segment_transition_ms": seg_tr, "compose_ms": comp,
            "schedule_on_one_gpu_ms": serial,
            "one_rank_of_8_path_ms": 2 * seg_fwd + seg_tr + comp,
            "note": "one_rank_of_8_path_ms sums a rank's own steps (prefill, transition, "
                    "compose, prefill from its entry state) and leaves out the all-gather "
                    "of the 8 (transition, exit state) pairs, 4 MiB each",
        }
        del cset, sq, sk, sv, sg, sb, Pm, Rm
        torch.cuda.empty_cache()

    if not args.no_decode:
        wd = kin.WORKLOADS["decode_256x32"]
        dd = kin.make_decode(wd.steps, wd.B, wd.H, wd.dk, wd.dv, dtype=wd.dtype, seed=wd.seed,
                             device=dev)
        state = dd["state"]
        dout = torch.empty((wd.B, wd.H, wd.dv), dtype=wd.dtype, device=dev)
        per_step = [dd[x].unbind(0) for x in ("q", "k", "v", "g", "beta")]

        def dstep(s):
            kda.kda_decode_step(per_step[0][s], per_step[1][s], per_step[2][s], per_step[3][s],
                                per_step[4][s], state, scale=wd.scale_value(), out=dout)

        for s in range(4):
            dstep(s)
        torch.cuda.synchronize()
        dev_ms = []
        walls = []
        for rep in range(args.decode_reps):
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(wd.steps)]
            torch.cuda.synchronize()
            tw = time.perf_counter()
            for s in range(wd.steps):
                evs[s][0].record(stream)
                dstep(s)
                evs[s][1].record(stream)
            torch.cuda.synchronize()
            walls.append(time.perf_counter() - tw)
            dev_ms += [a.elapsed_time(b) for a, b in evs]
        step_s = sum(dev_ms) / len(dev_ms) / 1e3
        sb, tb = decode_bytes(wd.B, wd.H, wd.dk, 2)
        result["decode"] = {
            "workload": "decode_256x32", "B": wd.B, "H": wd.H, "d": wd.dk,
            "steps_per_rep": wd.steps, "reps": args.decode_reps,
            "kernel_us_avg": step_s * 1e6,
            "state_GBps": sb / step_s / 1e9, "total_GBps": tb / step_s / 1e9,
            "hbm_frac": tb / step_s / 1e9 / HBM_PEAK_GBS,
            "wall_ms_per_64_steps": min(walls) * 1e3,
        }
        del dd, state
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        from oracle import oracle_forward  # the CPU baseline leg may load the oracle
        cores = max(1, min(os.cpu_count() or 1, 16))
        wcpu = kin.make_workload(w, device=dev)
        qc, kc, vc, gc, bc = (wcpu[x].cpu() for x in ("q", "k", "v", "g", "beta"))
        s0 = wcpu["initial_state"].cpu()
        # the whole workload (all B*H pairs at full length), repeated until about
        # 10 s of CPU work have been timed
        reps, cpu_s = 0, 0.0
        while reps < 1 or (cpu_s * cores < 10.0 and reps < 8):
            tc = time.perf_counter()
            oracle_forward(qc, kc, vc, gc, bc, scale, B=B, T=T, initial_state=s0,
                           store_out=True, nthreads=cores)
            cpu_s += time.perf_counter() - tc
            reps += 1
        result["cpu_baseline"] = {
            "value": reps * B * T / cpu_s, "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"the full prefill_4x4096 workload ({B * H} (sequence, head) pairs, "
                      f"T={T}) run {reps} times by the fp64 sequential recurrence with "
                      f"OpenMP over pairs: {cpu_s:.2f} s wall on {cores} threads",
        }
    print(json.dumps(result))


if __name__ == "__main__":
    main()
