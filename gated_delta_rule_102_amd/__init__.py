"""Kimi Delta Attention (KDA) for AMD Instinct MI355X (gfx950).

The compute path is ``libkda.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/kda.h``); :mod:`gated_delta_rule_102_amd.kda` is its thin
Python binding and :mod:`gated_delta_rule_102_amd.inputs` draws seeded inputs.
"""
from .kda import (  # noqa: F401
    KDAError,
    chunk_bwd,
    chunk_fwd_context_parallel,
    chunk_fwd,
    chunk_fwd_prologue,
    chunk_fwd_snapshots,
    chunk_fwd_varlen,
    decode_step,
    kda_abi_version,
    kda_chunk_bwd,
    kda_chunk_transition,
    kda_chunk_fwd,
    kda_chunk_fwd_prologue,
    kda_chunk_fwd_snapshots,
    kda_chunk_fwd_varlen,
    kda_decode_step,
    kda_state_compose,
    kda_status_string,
    load_library,
)
