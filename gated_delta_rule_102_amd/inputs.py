"""Seeded synthetic inputs for KDA prefill and decode.

This module holds no part of the KDA computation: it only draws random numbers
and shapes them into the distributions below, so that the HIP path and the CPU
oracle can be fed bit-identical tensors.  Both sides may import it; it imports
neither of them.

Distributions (one draw per element, fp32, in this fixed order from one
``torch.Generator`` seeded with ``seed``; for packed variable-length cases the
sequence lengths are drawn first):

  q, k   ~ N(0, 1), then L2-normalised over the key channels of each (token, head)
  v      ~ N(0, 1)
  g_raw  ~ N(0, 1);  g = max(-5, -softplus(g_raw))   (log-decay in [-5, 0))
  b_raw  ~ N(0, 1);  beta = sigmoid(b_raw)
  S0     ~ 0.1 * N(0, 1) in fp32 when a nonzero initial state is asked for

The -5 floor is the log-decay bound of the neurohive.io Kimi K3 review
(section "Sequence length: hybrid KDA and Gated MLA attention").  For the
"split decay" option, the first half of the heads get g = -5 everywhere and the
second half g ~ U(-0.05, 0): the two ends of the allowed decay range.  Lengths of
packed cases are log-uniform: L = floor(exp(U(ln lo, ln hi))), clipped to [lo, hi].

All tensors are cast to the requested dtype after the transforms; states stay fp32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

LOG_DECAY_FLOOR = -5.0


@dataclass(frozen=True)
class Workload:
    """A named synthetic workload.  ``kind`` is 'prefill', 'varlen' or 'decode'."""
    name: str
    kind: str
    dtype: torch.dtype
    H: int
    dk: int
    dv: int
    B: int = 1              # batch (prefill / decode)
    T: int = 0              # tokens per sequence (prefill)
    steps: int = 0          # decode steps
    nseq: int = 0           # sequences (varlen)
    len_range: tuple = (0, 0)
    nonzero_state: bool = False
    split_decay: bool = False
    scale: float = field(default=0.0)
    seed: int = 0

    def scale_value(self) -> float:
        return self.scale if self.scale else 1.0 / math.sqrt(self.dk)


# The five workloads the library is measured and checked on.
WORKLOADS = {
    "fp32_small": Workload("fp32_small", "prefill", torch.float32, H=2, dk=64, dv=64,
                           B=1, T=256, scale=1.0 / 8.0, seed=1000),
    "prefill_4x4096": Workload("prefill_4x4096", "prefill", torch.bfloat16, H=16, dk=128,
                               dv=128, B=4, T=4096, nonzero_state=True, seed=1001),
    "prefill_1x65536": Workload("prefill_1x65536", "prefill", torch.bfloat16, H=32, dk=128,
                                dv=128, B=1, T=65536, seed=1002),
    "decode_256x32": Workload("decode_256x32", "decode", torch.bfloat16, H=32, dk=128, dv=128,
                              B=256, steps=64, nonzero_state=True, seed=1003),
    "varlen_64seq": Workload("varlen_64seq", "varlen", torch.bfloat16, H=32, dk=128, dv=128,
                             nseq=64, len_range=(1024, 65536), split_decay=True, seed=1004),
}


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _unit(x):
    return x / x.norm(dim=-1, keepdim=True)


def draw_lengths(nseq, lo, hi, seed, device="cpu"):
    """Log-uniform sequence lengths in [lo, hi] (int64, on the CPU)."""
    gen = _gen("cpu", seed)
    u = torch.rand(nseq, generator=gen, dtype=torch.float64)
    L = torch.floor(torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo))))
    return L.clamp_(lo, hi).to(torch.int64)


def lengths_to_cu(lengths):
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.as_tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    return cu


def make_tokens(shape_qk, shape_v, shape_b, dtype, gen, device, split_decay=False,
                head_axis=-2):
    """Draw q, k, v, g, beta with the distributions of the module docstring."""
    f32 = torch.float32
    q = _unit(torch.randn(shape_qk, generator=gen, device=device, dtype=f32))
    k = _unit(torch.randn(shape_qk, generator=gen, device=device, dtype=f32))
    v = torch.randn(shape_v, generator=gen, device=device, dtype=f32)
    g_raw = torch.randn(shape_qk, generator=gen, device=device, dtype=f32)
    g = torch.clamp(-torch.nn.functional.softplus(g_raw), min=LOG_DECAY_FLOOR)
    b_raw = torch.randn(shape_b, generator=gen, device=device, dtype=f32)
    beta = torch.sigmoid(b_raw)
    if split_decay:
        H = shape_qk[head_axis]
        half = H // 2
        # uniform in (-0.05, 0] for the second half of the heads, -5 for the first
        idx = [slice(None)] * len(shape_qk)
        idx[head_axis % len(shape_qk)] = slice(half, H)
        u = torch.rand(g[tuple(idx)].shape, generator=gen, device=device, dtype=f32)
        g[tuple(idx)] = -0.05 * u
        idx[head_axis % len(shape_qk)] = slice(0, half)
        g[tuple(idx)] = LOG_DECAY_FLOOR
    return [x.to(dtype) for x in (q, k, v, g, beta)]


def make_prefill(B, T, H, dk, dv, dtype=torch.bfloat16, seed=0, device="cpu",
                 nonzero_state=False, split_decay=False):
    """Fixed-length prefill inputs: q, k, g [B,T,H,dk]; v [B,T,H,dv]; beta [B,T,H]."""
    gen = _gen(device, seed)
    q, k, v, g, beta = make_tokens((B, T, H, dk), (B, T, H, dv), (B, T, H), dtype, gen,
                                   device, split_decay=split_decay)
    s0 = None
    if nonzero_state:
        s0 = 0.1 * torch.randn((B, H, dk, dv), generator=gen, device=device,
                               dtype=torch.float32)
    return dict(q=q, k=k, v=v, g=g, beta=beta, initial_state=s0)


def make_prefill_raw(B, T, H, dk, dv, dtype=torch.bfloat16, seed=0, device="cpu",
                     nonzero_state=False, spread=2.0):
    """Raw activations for the fused prologue: q_raw, k_raw, g_raw [B,T,H,dk] and
    beta_raw [B,T,H] drawn N(0, spread^2) (q, k not normalised, gates not applied),
    v ~ N(0, 1), optional state ~ 0.1 N(0, 1).  Only random draws: the prologue's
    arithmetic is not done here."""
    gen = _gen(device, seed)
    f32 = torch.float32
    q = spread * torch.randn((B, T, H, dk), generator=gen, device=device, dtype=f32)
    k = spread * torch.randn((B, T, H, dk), generator=gen, device=device, dtype=f32)
    v = torch.randn((B, T, H, dv), generator=gen, device=device, dtype=f32)
    g = spread * torch.randn((B, T, H, dk), generator=gen, device=device, dtype=f32)
    b = spread * torch.randn((B, T, H), generator=gen, device=device, dtype=f32)
    s0 = None
    if nonzero_state:
        s0 = 0.1 * torch.randn((B, H, dk, dv), generator=gen, device=device, dtype=f32)
    return dict(q_raw=q.to(dtype), k_raw=k.to(dtype), v=v.to(dtype), g_raw=g.to(dtype),
                beta_raw=b.to(dtype), initial_state=s0)


def make_varlen(lengths, H, dk, dv, dtype=torch.bfloat16, seed=0, device="cpu",
                nonzero_state=False, split_decay=False):
    """Packed inputs [1, total_T, H, .] for the given sequence lengths."""
    lengths = [int(x) for x in lengths]
    total = sum(lengths)
    gen = _gen(device, seed)
    q, k, v, g, beta = make_tokens((1, total, H, dk), (1, total, H, dv), (1, total, H),
                                   dtype, gen, device, split_decay=split_decay)
    s0 = None
    if nonzero_state:
        s0 = 0.1 * torch.randn((len(lengths), H, dk, dv), generator=gen, device=device,
                               dtype=torch.float32)
    cu = lengths_to_cu(lengths).to(device)
    return dict(q=q, k=k, v=v, g=g, beta=beta, initial_state=s0, cu_seqlens=cu)


def make_cotangents(B, T, H, dk, dv, dtype=torch.bfloat16, seed=0, device="cpu",
                    final_state=True):
    """Cotangents for the backward: grad_out [B,T,H,dv] ~ N(0,1) in dtype and
    grad_final_state [B,H,dk,dv] ~ N(0,1) fp32 (or None)."""
    gen = _gen(device, seed)
    d_out = torch.randn((B, T, H, dv), generator=gen, device=device, dtype=torch.float32)
    d_fin = None
    if final_state:
        d_fin = torch.randn((B, H, dk, dv), generator=gen, device=device, dtype=torch.float32)
    return dict(grad_out=d_out.to(dtype), grad_final_state=d_fin)


def make_decode(steps, B, H, dk, dv, dtype=torch.bfloat16, seed=0, device="cpu"):
    """Decode inputs: per-step q, k, g [steps,B,H,dk]; v [steps,B,H,dv];
    beta [steps,B,H]; state [B,H,dk,dv] fp32 ~ 0.1 N(0,1)."""
    gen = _gen(device, seed)
    q, k, v, g, beta = make_tokens((steps, B, H, dk), (steps, B, H, dv), (steps, B, H),
                                   dtype, gen, device)
    s0 = 0.1 * torch.randn((B, H, dk, dv), generator=gen, device=device, dtype=torch.float32)
    return dict(q=q, k=k, v=v, g=g, beta=beta, state=s0)


def make_workload(w: Workload, device="cpu", **override):
    """Inputs for one of :data:`WORKLOADS` (fields may be overridden, e.g. B or T)."""
    if override:
        w = Workload(**{**w.__dict__, **override})
    if w.kind == "prefill":
        d = make_prefill(w.B, w.T, w.H, w.dk, w.dv, w.dtype, w.seed, device,
                         w.nonzero_state, w.split_decay)
    elif w.kind == "varlen":
        lengths = draw_lengths(w.nseq, w.len_range[0], w.len_range[1], w.seed)
        d = make_varlen(lengths.tolist(), w.H, w.dk, w.dv, w.dtype, w.seed + 1, device,
                        w.nonzero_state, w.split_decay)
        d["lengths"] = lengths
    elif w.kind == "decode":
        d = make_decode(w.steps, w.B, w.H, w.dk, w.dv, w.dtype, w.seed, device)
    else:
        raise ValueError(w.kind)
    d["scale"] = w.scale_value()
    return d
