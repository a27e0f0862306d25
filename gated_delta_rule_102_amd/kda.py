"""Thin ctypes binding over libkda.so with the same entry-point names as the C ABI.

This module only marshals arguments: it checks devices, dtypes, shapes and
contiguity, allocates outputs with PyTorch (device memory is PyTorch's job here),
and passes raw device pointers plus the current HIP stream to the library.
Every step of KDA runs in the library's HIP kernels.  There is no fallback: if
libkda.so is missing or the device is not gfx950, the calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_BF16, KDA_F32 = 0, 1
_lib = None

EXPORTS = ("kda_abi_version", "kda_status_string", "kda_chunk_fwd_schedule",
           "kda_chunk_fwd", "kda_chunk_fwd_workspace_size", "kda_chunk_fwd_ws",
           "kda_chunk_fwd_noalloc",
           "kda_prefill_workspace_size", "kda_prefill",
           "kda_chunk_fwd_prologue", "kda_chunk_fwd_snapshots",
           "kda_chunk_fwd_varlen", "kda_chunk_fwd_varlen_workspace_size", "kda_chunk_fwd_varlen_ws",
           "kda_chunk_fwd_varlen_prologue", "kda_chunk_fwd_varlen_snapshots",
           "kda_chunk_bwd", "kda_chunk_bwd_workspace_size", "kda_chunk_bwd_window_workspace_size",
           "kda_chunk_bwd_ws", "kda_chunk_bwd_varlen", "kda_chunk_bwd_varlen_workspace_size",
           "kda_chunk_bwd_varlen_window_workspace_size", "kda_chunk_bwd_varlen_ws",
           "kda_chunk_transition", "kda_chunk_transition_workspace_size", "kda_chunk_transition_ws",
           "kda_state_compose", "kda_decode_step", "kda_decode_step_prologue")


class PrefillDesc(ctypes.Structure):
    """ctypes mirror of ``kda_prefill_desc`` (include/kda.h)."""
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p),
                ("initial_state", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("final_state", ctypes.c_void_p), ("cu_seqlens", ctypes.c_void_p),
                ("N", ctypes.c_int), ("T", ctypes.c_int), ("total_T", ctypes.c_int),
                ("H", ctypes.c_int), ("dk", ctypes.c_int), ("dv", ctypes.c_int),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int), ("prologue", ctypes.c_int),
                ("snapshots", ctypes.c_void_p), ("snapshot_tokens", ctypes.c_int)]


class KDAError(RuntimeError):
    """A non-zero status returned by libkda.so."""

    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")
        self.status = status


def load_library(path: str = LIB_PATH):
    """Load libkda.so (built in-tree by ``python -m gated_delta_rule_102_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m gated_delta_rule_102_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.kda_abi_version.argtypes = []
    lib.kda_abi_version.restype = i32
    lib.kda_status_string.argtypes = [i32]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                  f32, i32, vp]
    lib.kda_chunk_fwd.restype = i32
    lib.kda_chunk_fwd_schedule.argtypes = [i32] * 8
    lib.kda_chunk_fwd_schedule.restype = ctypes.c_char_p
    lib.kda_chunk_fwd_workspace_size.argtypes = [i32] * 6
    lib.kda_chunk_fwd_workspace_size.restype = ctypes.c_size_t
    lib.kda_chunk_fwd_ws.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                     f32, i32, vp, ctypes.c_size_t, vp]
    lib.kda_chunk_fwd_ws.restype = i32
    lib.kda_chunk_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                          f32, i32, vp]
    lib.kda_chunk_fwd_noalloc.restype = i32
    sz = ctypes.c_size_t
    lib.kda_prefill_workspace_size.argtypes = [ctypes.POINTER(PrefillDesc), ctypes.POINTER(sz)]
    lib.kda_prefill_workspace_size.restype = i32
    lib.kda_prefill.argtypes = [ctypes.POINTER(PrefillDesc), vp, sz, vp]
    lib.kda_prefill.restype = i32
    lib.kda_chunk_fwd_varlen_workspace_size.argtypes = [i32] * 6
    lib.kda_chunk_fwd_varlen_workspace_size.restype = sz
    lib.kda_chunk_fwd_varlen_ws.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                            i32, i32, f32, i32, vp, sz, vp]
    lib.kda_chunk_fwd_varlen_ws.restype = i32
    lib.kda_chunk_bwd_workspace_size.argtypes = [i32] * 6
    lib.kda_chunk_bwd_workspace_size.restype = sz
    lib.kda_chunk_bwd_window_workspace_size.argtypes = [i32] * 7
    lib.kda_chunk_bwd_window_workspace_size.restype = sz
    lib.kda_chunk_bwd_ws.argtypes = [vp] * 14 + [i32, i32, i32, i32, i32, f32, i32, vp, sz, vp]
    lib.kda_chunk_bwd_ws.restype = i32
    lib.kda_chunk_bwd_varlen_workspace_size.argtypes = [i32] * 6
    lib.kda_chunk_bwd_varlen_workspace_size.restype = sz
    lib.kda_chunk_bwd_varlen_window_workspace_size.argtypes = [i32] * 7
    lib.kda_chunk_bwd_varlen_window_workspace_size.restype = sz
    lib.kda_chunk_bwd_varlen_ws.argtypes = [vp] * 15 + [i32, i32, i32, i32, i32, f32, i32, vp, sz,
                                                        vp]
    lib.kda_chunk_bwd_varlen_ws.restype = i32
    lib.kda_chunk_transition_workspace_size.argtypes = [i32] * 6
    lib.kda_chunk_transition_workspace_size.restype = sz
    lib.kda_chunk_transition_ws.argtypes = [vp] * 5 + [i32] * 6 + [vp, sz, vp]
    lib.kda_chunk_transition_ws.restype = i32
    lib.kda_chunk_fwd_prologue.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                           i32, f32, i32, vp]
    lib.kda_chunk_fwd_prologue.restype = i32
    lib.kda_chunk_fwd_snapshots.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                            i32, i32, i32, f32, i32, vp]
    lib.kda_chunk_fwd_snapshots.restype = i32
    lib.kda_chunk_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                         i32, i32, f32, i32, vp]
    lib.kda_chunk_fwd_varlen.restype = i32
    lib.kda_chunk_fwd_varlen_prologue.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32,
                                                  i32, i32, i32, f32, i32, vp]
    lib.kda_chunk_fwd_varlen_prologue.restype = i32
    lib.kda_chunk_fwd_varlen_snapshots.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp,
                                                   i32, i32, i32, i32, i32, f32, i32, vp]
    lib.kda_chunk_fwd_varlen_snapshots.restype = i32
    lib.kda_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp]
    lib.kda_decode_step.restype = i32
    lib.kda_decode_step_prologue.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32,
                                             i32, vp]
    lib.kda_decode_step_prologue.restype = i32
    lib.kda_chunk_bwd.argtypes = [vp] * 14 + [i32, i32, i32, i32, i32, f32, i32, vp]
    lib.kda_chunk_bwd.restype = i32
    lib.kda_chunk_bwd_varlen.argtypes = [vp] * 15 + [i32, i32, i32, i32, i32, f32, i32, vp]
    lib.kda_chunk_bwd_varlen.restype = i32
    lib.kda_chunk_transition.argtypes = [vp] * 5 + [i32] * 6 + [vp]
    lib.kda_chunk_transition.restype = i32
    lib.kda_state_compose.argtypes = [vp] * 4 + [i32] * 5 + [vp]
    lib.kda_state_compose.restype = i32
    _lib = lib
    return lib


def kda_abi_version() -> int:
    return load_library().kda_abi_version()


def status_string(status: int) -> str:
    return load_library().kda_status_string(int(status)).decode()


kda_status_string = status_string


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"KDA inputs must be bfloat16 or float32, got {t.dtype}")


def _check(ts, dtype, device):
    for name, t in ts.items():
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")
        if t.dtype != dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _check_state(name, t, shape, device):
    if t is None:
        return
    if t.device != device or t.dtype != torch.float32 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor on {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_out(t, shape, dtype, device):
    """A caller-supplied output must match exactly: the kernels size their stores from
    the call's sizes, not from the tensor."""
    _check(dict(out=t), dtype, device)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"out has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _raise(fn, rc):
    if rc != 0:
        raise KDAError(fn, rc)


def prefill_schedule_name(N, T, H, d, dtype=torch.bfloat16, varlen=False, total_T=0):
    """Kernels a prefill call with these sizes launches (kda_chunk_fwd_schedule)."""
    code = KDA_BF16 if dtype == torch.bfloat16 else KDA_F32
    return load_library().kda_chunk_fwd_schedule(int(N), int(T), int(total_T or N * max(T, 1)),
                                                 int(H), int(d), int(d), code,
                                                 1 if varlen else 0).decode()


kda_chunk_fwd_schedule = prefill_schedule_name


def kda_chunk_fwd_workspace_size(B, T, H, dk, dv, dtype=torch.bfloat16) -> int:
    """Workspace bytes kda_chunk_fwd_ws needs for these sizes (0: sizes not accepted)."""
    code = KDA_BF16 if dtype == torch.bfloat16 else KDA_F32 if dtype == torch.float32 else -1
    return int(load_library().kda_chunk_fwd_workspace_size(B, T, H, dk, dv, code))


def _ws_arg(workspace, device):
    """(pointer, bytes) of a caller workspace tensor, 256-byte aligned inside it."""
    if workspace.device != device or workspace.dtype != torch.uint8:
        raise ValueError(f"workspace must be a uint8 tensor on {device}")
    base = workspace.data_ptr()
    off = (-base) % 256
    return ctypes.c_void_p(base + off), max(workspace.numel() - off, 0)


def _ws_tensor(nbytes, device):
    """A uint8 device tensor with room for `nbytes` at a 256-byte aligned offset."""
    return torch.empty(int(nbytes) + 256, dtype=torch.uint8, device=device)


def chunk_fwd_workspace(q, v):
    """A uint8 device tensor large enough to serve as the workspace of prefill calls
    shaped like (q, v) (256 bytes of slack only when the call needs none); allocated
    once and passed as ``workspace=`` to kda_chunk_fwd."""
    B, T, H, dk = q.shape
    d = PrefillDesc(q=256, k=256, v=256, g=256, beta=256, out=256, N=B, T=T, H=H, dk=dk,
                    dv=v.shape[-1], scale=1.0, dtype=_dtype_code(q))
    return _ws_tensor(prefill_workspace_size(d), q.device)


def varlen_workspace(q, v, cu_seqlens):
    """Workspace tensor for kda_chunk_fwd_varlen calls shaped like (q, v, cu_seqlens)."""
    H, dk = q.shape[-2], q.shape[-1]
    n = load_library().kda_chunk_fwd_varlen_workspace_size(
        cu_seqlens.numel() - 1, q.numel() // (H * dk), H, dk, v.shape[-1], _dtype_code(q))
    return _ws_tensor(n, q.device)


def prefill_workspace_size(desc):
    """Bytes of workspace kda_prefill needs for a PrefillDesc (raises on bad arguments)."""
    n = ctypes.c_size_t(0)
    _raise("kda_prefill_workspace_size",
           load_library().kda_prefill_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return int(n.value)


def kda_prefill(q, k, v, g, beta, scale=None, initial_state=None, cu_seqlens=None,
                prologue=False, snapshot_tokens=0, output_final_state=True, out=None,
                final_state=None, snapshots=None, workspace=None):
    """Every prefill variant through the descriptor entry point kda_prefill, on a
    caller workspace: fixed length ([B,T,H,.] tensors) or packed (``cu_seqlens``,
    [1,total_T,H,.] or [total_T,H,.]), raw activations (``prologue``), snapshots every
    ``snapshot_tokens`` tokens.  ``workspace`` None: a torch tensor of the size the
    library asks for.  Returns ``(out, final_state, snapshots)``."""
    lib = load_library()
    packed = cu_seqlens is not None
    H, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    dtype, device = q.dtype, q.device
    _check(dict(q=q, k=k, v=v, g=g, beta=beta), dtype, device)
    if packed:
        H, dk, dv, total_T, N, out, final_state = _varlen_prep(
            q, k, v, g, beta, cu_seqlens, initial_state, output_final_state, out, final_state)
        T = 0
        if snapshot_tokens:
            rows = varlen_snapshot_rows(cu_seqlens, snapshot_tokens)
            shape = (int(rows[-1]), H, dk, dv)
    else:
        N, T = q.shape[0], q.shape[1]
        total_T = N * T
        if k.shape != q.shape or g.shape != q.shape or v.shape[:3] != q.shape[:3] \
                or beta.shape != q.shape[:3]:
            raise ValueError("shape mismatch among q, k, v, g, beta")
        _check_state("initial_state", initial_state, (N, H, dk, dv), device)
        if out is None:
            out = torch.empty((N, T, H, dv), dtype=dtype, device=device)
        _check_out(out, (N, T, H, dv), dtype, device)
        if final_state is None and output_final_state:
            final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=device)
        _check_state("final_state", final_state, (N, H, dk, dv), device)
        if snapshot_tokens:
            shape = (N, H, -(-T // snapshot_tokens), dk, dv)
    if snapshot_tokens:
        if snapshots is None:
            snapshots = torch.empty(shape, dtype=torch.float32, device=device)
        _check_state("snapshots", snapshots, shape, device)
    scale = 1.0 / math.sqrt(dk) if scale is None else float(scale)
    d = PrefillDesc(q=q.data_ptr(), k=k.data_ptr(), v=v.data_ptr(), g=g.data_ptr(),
                    beta=beta.data_ptr(),
                    initial_state=None if initial_state is None else initial_state.data_ptr(),
                    out=out.data_ptr(),
                    final_state=None if final_state is None else final_state.data_ptr(),
                    cu_seqlens=cu_seqlens.contiguous().data_ptr() if packed else None,
                    N=N, T=T, total_T=total_T, H=H, dk=dk, dv=dv, scale=scale,
                    dtype=_dtype_code(q), prologue=1 if prologue else 0,
                    snapshots=None if snapshots is None else snapshots.data_ptr(),
                    snapshot_tokens=int(snapshot_tokens))
    if workspace is None:
        workspace = _ws_tensor(prefill_workspace_size(d), device)
    wp, wn = _ws_arg(workspace, device)
    _raise("kda_prefill", lib.kda_prefill(ctypes.byref(d), wp, wn, _stream(q)))
    return out, final_state, snapshots


def kda_chunk_fwd(q, k, v, g, beta, scale=None, initial_state=None, output_final_state=True,
                  out=None, final_state=None, workspace=None):
    """Chunked prefill.  q, k, g: [B,T,H,dk]; v: [B,T,H,dv]; beta: [B,T,H].

    Returns ``(out [B,T,H,dv], final_state [B,H,dk,dv] fp32 or None)``.
    ``final_state`` may be passed (and may be ``initial_state`` for in-place use).
    With ``workspace`` (a device uint8 tensor from ``chunk_fwd_workspace``) the call
    goes to kda_chunk_fwd_ws and allocates nothing; without it, to kda_chunk_fwd.
    """
    lib = load_library()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dtype, device = q.dtype, q.device
    _check(dict(q=q, k=k, v=v, g=g, beta=beta), dtype, device)
    if k.shape != q.shape or g.shape != q.shape or v.shape[:3] != q.shape[:3] \
            or beta.shape != q.shape[:3]:
        raise ValueError("shape mismatch among q, k, v, g, beta")
    _check_state("initial_state", initial_state, (B, H, dk, dv), device)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=dtype, device=device)
    _check_out(out, (B, T, H, dv), dtype, device)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=device)
    _check_state("final_state", final_state, (B, H, dk, dv), device)
    scale = 1.0 / math.sqrt(dk) if scale is None else float(scale)
    if workspace is not None:
        wp, wn = _ws_arg(workspace, device)
        rc = lib.kda_chunk_fwd_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                  _ptr(initial_state), _ptr(out), _ptr(final_state), B, T, H, dk,
                                  dv, scale, _dtype_code(q), wp, wn, _stream(q))
        _raise("kda_chunk_fwd_ws", rc)
        return out, final_state
    rc = lib.kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                           _ptr(out), _ptr(final_state), B, T, H, dk, dv, scale,
                           _dtype_code(q), _stream(q))
    _raise("kda_chunk_fwd", rc)
    return out, final_state


def kda_chunk_fwd_noalloc(q, k, v, g, beta, scale=None, initial_state=None,
                          output_final_state=True, out=None, final_state=None):
    """kda_chunk_fwd through kda_chunk_fwd_noalloc, which allocates nothing: its
    scratch is the library's fixed 64 MiB per-GPU array (calls that overlap on one GPU
    race on it).  Sizes whose windows do not fit raise KDAError (KDA_ERR_WORKSPACE).
    Outputs are allocated here when not given, as for kda_chunk_fwd."""
    lib = load_library()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dtype, device = q.dtype, q.device
    _check(dict(q=q, k=k, v=v, g=g, beta=beta), dtype, device)
    if k.shape != q.shape or g.shape != q.shape or v.shape[:3] != q.shape[:3] \
            or beta.shape != q.shape[:3]:
        raise ValueError("shape mismatch among q, k, v, g, beta")
    _check_state("initial_state", initial_state, (B, H, dk, dv), device)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=dtype, device=device)
    _check_out(out, (B, T, H, dv), dtype, device)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=device)
    _check_state("final_state", final_state, (B, H, dk, dv), device)
    scale = 1.0 / math.sqrt(dk) if scale is None else float(scale)
    rc = lib.kda_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                   _ptr(initial_state), _ptr(out), _ptr(final_state), B, T, H, dk,
                                   dv, scale, _dtype_code(q), _stream(q))
    _raise("kda_chunk_fwd_noalloc", rc)
    return out, final_state


def kda_chunk_fwd_prologue(q_raw, k_raw, v, g_raw, beta_raw, scale=None, initial_state=None,
                           output_final_state=True, out=None, final_state=None):
    """kda_chunk_fwd on raw activations: the kernels normalise q and k (unit L2 norm
    per token and head), form g = max(-5, -softplus(g_raw)) and beta =
    sigmoid(beta_raw) while loading them.  Shapes as for kda_chunk_fwd."""
    lib = load_library()
    B, T, H, dk = q_raw.shape
    dv = v.shape[-1]
    dtype, device = q_raw.dtype, q_raw.device
    _check(dict(q_raw=q_raw, k_raw=k_raw, v=v, g_raw=g_raw, beta_raw=beta_raw), dtype, device)
    if k_raw.shape != q_raw.shape or g_raw.shape != q_raw.shape or v.shape[:3] != q_raw.shape[:3] \
            or beta_raw.shape != q_raw.shape[:3]:
        raise ValueError("shape mismatch among q_raw, k_raw, v, g_raw, beta_raw")
    _check_state("initial_state", initial_state, (B, H, dk, dv), device)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=dtype, device=device)
    _check_out(out, (B, T, H, dv), dtype, device)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=device)
    _check_state("final_state", final_state, (B, H, dk, dv), device)
    scale = 1.0 / math.sqrt(dk) if scale is None else float(scale)
    rc = lib.kda_chunk_fwd_prologue(_ptr(q_raw), _ptr(k_raw), _ptr(v), _ptr(g_raw),
                                    _ptr(beta_raw), _ptr(initial_state), _ptr(out),
                                    _ptr(final_state), B, T, H, dk, dv, scale,
                                    _dtype_code(q_raw), _stream(q_raw))
    _raise("kda_chunk_fwd_prologue", rc)
    return out, final_state


def kda_chunk_fwd_snapshots(q, k, v, g, beta, scale=None, initial_state=None,
                            snapshot_tokens=512, output_final_state=True, out=None,
                            final_state=None, snapshots=None):
    """kda_chunk_fwd that also returns the state after every ``snapshot_tokens``
    tokens (a multiple of 64) and at the end.  Returns ``(out, final_state,
    snapshots [B,H,ceil(T/snapshot_tokens),dk,dv] fp32)``."""
    lib = load_library()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dtype, device = q.dtype, q.device
    _check(dict(q=q, k=k, v=v, g=g, beta=beta), dtype, device)
    if k.shape != q.shape or g.shape != q.shape or v.shape[:3] != q.shape[:3] \
            or beta.shape != q.shape[:3]:
        raise ValueError("shape mismatch among q, k, v, g, beta")
    _check_state("initial_state", initial_state, (B, H, dk, dv), device)
    snapshot_tokens = int(snapshot_tokens)
    nsnap = -(-T // snapshot_tokens) if snapshot_tokens > 0 else 0
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=dtype, device=device)
    _check_out(out, (B, T, H, dv), dtype, device)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=device)
    _check_state("final_state", final_state, (B, H, dk, dv), device)
    if snapshots is None and nsnap > 0:
        snapshots = torch.empty((B, H, nsnap, dk, dv), dtype=torch.float32, device=device)
    _check_state("snapshots", snapshots, (B, H, nsnap, dk, dv), device)
    scale = 1.0 / math.sqrt(dk) if scale is None else float(scale)
    rc = lib.kda_chunk_fwd_snapshots(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                     _ptr(initial_state), _ptr(out), _ptr(final_state),
                                     _ptr(snapshots), snapshot_tokens, B, T, H, dk, dv, scale,
                                     _dtype_code(q), _stream(q))
    _raise("kda_chunk_fwd_snapshots", rc)
    return out, final_state, snapshots


def _varlen_prep(q, k, v, g, beta, cu_seqlens, initial_state, output_final_state, out,
                 final_state):
    H, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    total_T = q.numel() // (H * dk)
    N = cu_seqlens.numel() - 1
    dtype, device = q.dtype, q.device
    _check(dict(q=q, k=k, v=v, g=g, beta=beta), dtype, device)
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.device != device:
        raise ValueError("cu_seqlens must be int32 on the same device")
    if k.shape != q.shape or g.shape != q.shape or v.numel() != total_T * H * dv \
            or beta.numel() != total_T * H:
        raise ValueError("shape mismatch among q, k, v, g, beta")
    _check_state("initial_state", initial_state, (N, H, dk, dv), device)
    if out is None:
        out = torch.empty(v.shape, dtype=dtype, device=device)
    _check_out(out, v.shape, dtype, device)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=device)
    _check_state("final_state", final_state, (N, H, dk, dv), device)
    return H, dk, dv, total_T, N, out, final_state


def kda_chunk_fwd_varlen(q, k, v, g, beta, cu_seqlens, scale=None, initial_state=None,
                         output_final_state=True, out=None, final_state=None, workspace=None):
    """Packed variable-length prefill.  q, k, g: [1,total_T,H,dk] (or [total_T,H,dk]);
    cu_seqlens: int32 [N+1] on the device.  Returns ``(out, final_state [N,H,dk,dv])``.
    With ``workspace`` (a tensor from ``varlen_workspace``) the call goes to
    kda_chunk_fwd_varlen_ws and allocates nothing."""
    lib = load_library()
    H, dk, dv, total_T, N, out, final_state = _varlen_prep(
        q, k, v, g, beta, cu_seqlens, initial_state, output_final_state, out, final_state)
    scale = 1.0 / math.sqrt(dk) if scale is None else float(scale)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(out),
            _ptr(final_state), _ptr(cu_seqlens.contiguous()), N, total_T, H, dk, dv, scale,
            _dtype_code(q))
    if workspace is not None:
        wp, wn = _ws_arg(workspace, q.device)
        _raise("kda_chunk_fwd_varlen_ws", lib.kda_chunk_fwd_varlen_ws(*args, wp, wn, _stream(q)))
        return out, final_state
    _raise("kda_chunk_fwd_varlen", lib.kda_chunk_fwd_varlen(*args, _stream(q)))
    return out, final_state


def kda_chunk_fwd_varlen_prologue(q_raw, k_raw, v, g_raw, beta_raw, cu_seqlens, scale=None,
                                  initial_state=None, output_final_state=True, out=None,
                                  final_state=None):
    """kda_chunk_fwd_varlen on raw activations with the fused gate/normalisation
    prologue (see kda_chunk_fwd_prologue)."""
    lib = load_library()
    H, dk, dv, total_T, N, out, final_state = _varlen_prep(
        q_raw, k_raw, v, g_raw, beta_raw, cu_seqlens, initial_state, output_final_state, out,
        final_state)
    scale = 1.0 / math.sqrt(dk) if scale is None else float(scale)
    rc = lib.kda_chunk_fwd_varlen_prologue(_ptr(q_raw), _ptr(k_raw), _ptr(v), _ptr(g_raw),
                                           _ptr(beta_raw), _ptr(initial_state), _ptr(out),
                                           _ptr(final_state), _ptr(cu_seqlens.contiguous()), N,
                                           total_T, H, dk, dv, scale, _dtype_code(q_raw),
                                           _stream(q_raw))
    _raise("kda_chunk_fwd_varlen_prologue", rc)
    return out, final_state


def varlen_snapshot_rows(cu_seqlens, snapshot_tokens):
    """Per-sequence first snapshot row (int64 [N+1], host) of the varlen snapshot layout:
    sequence n owns rows [rows[n], rows[n+1]), ceil(L_n / snapshot_tokens) of them."""
    lengths = (cu_seqlens[1:] - cu_seqlens[:-1]).to("cpu", torch.int64).clamp_(min=0)
    per = (lengths + snapshot_tokens - 1) // snapshot_tokens
    return torch.cat([torch.zeros(1, dtype=torch.int64), torch.cumsum(per, 0)])


def kda_chunk_fwd_varlen_snapshots(q, k, v, g, beta, cu_seqlens, scale=None, initial_state=None,
                                   snapshot_tokens=512, output_final_state=True, out=None,
                                   final_state=None, snapshots=None):
    """kda_chunk_fwd_varlen that also returns each sequence's state every
    ``snapshot_tokens`` tokens.  Returns ``(out, final_state, snapshots [S_total,H,dk,dv],
    rows)`` with ``rows = varlen_snapshot_rows(cu_seqlens, snapshot_tokens)`` (reads the
    lengths back to the host to size the snapshot buffer)."""
    lib = load_library()
    H, dk, dv, total_T, N, out, final_state = _varlen_prep(
        q, k, v, g, beta, cu_seqlens, initial_state, output_final_state, out, final_state)
    if snapshot_tokens <= 0 or snapshot_tokens % 64 != 0:
        raise ValueError("snapshot_tokens must be a positive multiple of 64")
    rows = varlen_snapshot_rows(cu_seqlens, snapshot_tokens)
    shape = (int(rows[-1]), H, dk, dv)
    if snapshots is None:
        snapshots = torch.empty(shape, dtype=torch.float32, device=q.device)
    _check_state("snapshots", snapshots, shape, q.device)
    scale = 1.0 / math.sqrt(dk) if scale is None else float(scale)
    rc = lib.kda_chunk_fwd_varlen_snapshots(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                            _ptr(initial_state), _ptr(out), _ptr(final_state),
                                            _ptr(snapshots), int(snapshot_tokens),
                                            _ptr(cu_seqlens.contiguous()), N, total_T, H, dk,
                                            dv, scale, _dtype_code(q), _stream(q))
    _raise("kda_chunk_fwd_varlen_snapshots", rc)
    return out, final_state, snapshots, rows


def _decode(fn, q, k, v, g, beta, state, scale, out):
    lib = load_library()
    B, H, dk = q.shape
    dv = v.shape[-1]
    dtype, device = q.dtype, q.device
    _check(dict(q=q, k=k, v=v, g=g, beta=beta), dtype, device)
    if k.shape != q.shape or g.shape != q.shape or v.shape[:2] != q.shape[:2] \
            or beta.shape != q.shape[:2]:
        raise ValueError("shape mismatch among q, k, v, g, beta")
    _check_state("state", state, (B, H, dk, dv), device)
    if out is None:
        out = torch.empty((B, H, dv), dtype=dtype, device=device)
    _check_out(out, (B, H, dv), dtype, device)
    scale = 1.0 / math.sqrt(dk) if scale is None else float(scale)
    rc = getattr(lib, fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state),
                          _ptr(out), B, H, dk, dv, scale, _dtype_code(q), _stream(q))
    _raise(fn, rc)
    return out


def kda_decode_step(q, k, v, g, beta, state, scale=None, out=None):
    """One decode token.  q, k, g: [B,H,dk]; v: [B,H,dv]; beta: [B,H];
    state: [B,H,dk,dv] fp32, updated in place.  Returns out [B,H,dv]."""
    return _decode("kda_decode_step", q, k, v, g, beta, state, scale, out)


def kda_decode_step_prologue(q_raw, k_raw, v, g_raw, beta_raw, state, scale=None, out=None):
    """kda_decode_step on raw activations with the fused gate/normalisation prologue."""
    return _decode("kda_decode_step_prologue", q_raw, k_raw, v, g_raw, beta_raw, state, scale,
                   out)


def kda_chunk_bwd(q, k, v, g, beta, grad_out, scale=None, initial_state=None,
                  grad_final_state=None, need_initial_state_grad=True, workspace=None):
    """Gradients of sum(grad_out * out) + sum(grad_final_state * final_state) for
    kda_chunk_fwd's inputs (same shapes and dtype).  Returns ``(grad_q, grad_k,
    grad_v, grad_g, grad_beta, grad_initial_state or None)``; the initial-state
    gradient is fp32 [B,H,dk,dv].  With ``workspace`` (``chunk_bwd_workspace``) the call
    goes to kda_chunk_bwd_ws and allocates nothing."""
    lib = load_library()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dtype, device = q.dtype, q.device
    _check(dict(q=q, k=k, v=v, g=g, beta=beta, grad_out=grad_out), dtype, device)
    if k.shape != q.shape or g.shape != q.shape or v.shape[:3] != q.shape[:3] \
            or beta.shape != q.shape[:3] or grad_out.shape != v.shape:
        raise ValueError("shape mismatch among q, k, v, g, beta, grad_out")
    _check_state("initial_state", initial_state, (B, H, dk, dv), device)
    _check_state("grad_final_state", grad_final_state, (B, H, dk, dv), device)
    grads = [torch.empty_like(x) for x in (q, k, v, g, beta)]
    ds0 = torch.empty((B, H, dk, dv), dtype=torch.float32, device=device) \
        if need_initial_state_grad else None
    scale = 1.0 / math.sqrt(dk) if scale is None else float(scale)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(grad_out),
            _ptr(grad_final_state), *(_ptr(x) for x in grads), _ptr(ds0), B, T, H, dk, dv, scale,
            _dtype_code(q))
    if workspace is not None:
        wp, wn = _ws_arg(workspace, device)
        _raise("kda_chunk_bwd_ws", lib.kda_chunk_bwd_ws(*args, wp, wn, _stream(q)))
    else:
        _raise("kda_chunk_bwd", lib.kda_chunk_bwd(*args, _stream(q)))
    return (*grads, ds0)


def chunk_bwd_workspace(q, v, window_chunks=0):
    """Workspace tensor for kda_chunk_bwd calls shaped like (q [B,T,H,dk], v): the
    one-pass size, or with ``window_chunks`` > 0 the size of windows of that many chunks
    (a call given it runs in such windows)."""
    B, T, H, dk = q.shape
    n = load_library().kda_chunk_bwd_window_workspace_size(B, T, H, dk, v.shape[-1], _dtype_code(q),
                                                           int(window_chunks))
    if n == 0:
        raise ValueError("backward sizes not accepted by the library")
    return _ws_tensor(n, q.device)


def chunk_bwd_varlen_workspace(q, v, cu_seqlens, window_chunks=0):
    """Workspace tensor for kda_chunk_bwd_varlen calls shaped like (q, v, cu_seqlens),
    one-pass or for windows of ``window_chunks`` chunks."""
    H, dk = q.shape[-2], q.shape[-1]
    n = load_library().kda_chunk_bwd_varlen_window_workspace_size(
        cu_seqlens.numel() - 1, q.numel() // (H * dk), H, dk, v.shape[-1], _dtype_code(q),
        int(window_chunks))
    if n == 0:
        raise ValueError("backward sizes not accepted by the library")
    return _ws_tensor(n, q.device)


def kda_chunk_bwd_varlen(q, k, v, g, beta, grad_out, cu_seqlens, scale=None, initial_state=None,
                         grad_final_state=None, need_initial_state_grad=True, workspace=None):
    """kda_chunk_bwd for packed sequences (layouts of kda_chunk_fwd_varlen: q, k, g
    [1,total_T,H,dk] or [total_T,H,dk]; cu_seqlens int32 [N+1] on the device).
    Returns ``(grad_q, grad_k, grad_v, grad_g, grad_beta, grad_initial_state [N,H,dk,dv]
    or None)``; token gradients outside every sequence are zero."""
    lib = load_library()
    H, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    total_T = q.numel() // (H * dk)
    N = cu_seqlens.numel() - 1
    dtype, device = q.dtype, q.device
    _check(dict(q=q, k=k, v=v, g=g, beta=beta, grad_out=grad_out), dtype, device)
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.device != device:
        raise ValueError("cu_seqlens must be int32 on the same device")
    if k.shape != q.shape or g.shape != q.shape or v.numel() != total_T * H * dv \
            or beta.numel() != total_T * H or grad_out.shape != v.shape:
        raise ValueError("shape mismatch among q, k, v, g, beta, grad_out")
    _check_state("initial_state", initial_state, (N, H, dk, dv), device)
    _check_state("grad_final_state", grad_final_state, (N, H, dk, dv), device)
    grads = [torch.zeros_like(x) for x in (q, k, v, g, beta)]
    ds0 = torch.empty((N, H, dk, dv), dtype=torch.float32, device=device) \
        if need_initial_state_grad else None
    scale = 1.0 / math.sqrt(dk) if scale is None else float(scale)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(grad_out),
            _ptr(grad_final_state), *(_ptr(x) for x in grads), _ptr(ds0),
            _ptr(cu_seqlens.contiguous()), N, total_T, H, dk, dv, scale, _dtype_code(q))
    if workspace is not None:
        wp, wn = _ws_arg(workspace, device)
        _raise("kda_chunk_bwd_varlen_ws", lib.kda_chunk_bwd_varlen_ws(*args, wp, wn, _stream(q)))
    else:
        _raise("kda_chunk_bwd_varlen", lib.kda_chunk_bwd_varlen(*args, _stream(q)))
    return (*grads, ds0)


def transition_workspace(q):
    """Workspace tensor for kda_chunk_transition calls shaped like q [B,T,H,dk]."""
    B, T, H, dk = q.shape
    n = load_library().kda_chunk_transition_workspace_size(B, T, H, dk, dk, _dtype_code(q))
    if n == 0:
        raise ValueError("transition sizes not accepted by the library")
    return _ws_tensor(n, q.device)


def kda_chunk_transition(q, k, g, beta, transition=None, workspace=None):
    """Transition of each of B segments: the exit state with v = 0 from the identity,
    P [B,H,dk,dk] fp32 (so that S_exit = P S_entry + the zero-entry exit state)."""
    lib = load_library()
    B, T, H, dk = q.shape
    dtype, device = q.dtype, q.device
    _check(dict(q=q, k=k, g=g, beta=beta), dtype, device)
    if k.shape != q.shape or g.shape != q.shape or beta.shape != q.shape[:3]:
        raise ValueError("shape mismatch among q, k, g, beta")
    if transition is None:
        transition = torch.empty((B, H, dk, dk), dtype=torch.float32, device=device)
    _check_state("transition", transition, (B, H, dk, dk), device)
    args = (_ptr(q), _ptr(k), _ptr(g), _ptr(beta), _ptr(transition), B, T, H, dk, dk,
            _dtype_code(q))
    if workspace is not None:
        wp, wn = _ws_arg(workspace, device)
        _raise("kda_chunk_transition_ws", lib.kda_chunk_transition_ws(*args, wp, wn, _stream(q)))
    else:
        _raise("kda_chunk_transition", lib.kda_chunk_transition(*args, _stream(q)))
    return transition


def kda_state_compose(transitions, partial_states, initial_state=None, entry_states=None):
    """Entry state of every segment: transitions [R,B,H,dk,dk] and partial_states
    [R,B,H,dk,dv] fp32 -> entry_states [R+1,B,H,dk,dv] with entry[0] = initial_state
    (zero if None) and entry[r+1] = transitions[r] @ entry[r] + partial_states[r]."""
    lib = load_library()
    R, B, H, dk, _ = transitions.shape
    dv = partial_states.shape[-1]
    device = transitions.device
    _check_state("transitions", transitions, (R, B, H, dk, dk), device)
    _check_state("partial_states", partial_states, (R, B, H, dk, dv), device)
    _check_state("initial_state", initial_state, (B, H, dk, dv), device)
    if entry_states is None:
        entry_states = torch.empty((R + 1, B, H, dk, dv), dtype=torch.float32, device=device)
    _check_state("entry_states", entry_states, (R + 1, B, H, dk, dv), device)
    rc = lib.kda_state_compose(_ptr(transitions), _ptr(partial_states), _ptr(initial_state),
                               _ptr(entry_states), R, B, H, dk, dv, _stream(transitions))
    _raise("kda_state_compose", rc)
    return entry_states


def chunk_fwd_context_parallel(q, k, v, g, beta, segment_tokens, scale=None,
                               initial_state=None):
    """kda_chunk_fwd over segments of ``segment_tokens`` tokens scheduled as context
    parallelism would place them on several GPUs, here all on q's device:
      1. every segment (independent): its exit state from a zero entry state
         (kda_chunk_fwd) and its transition (kda_chunk_transition);
      2. the entry state of every segment (kda_state_compose) -- across GPUs this
         is where the per-segment (transition, exit state) pairs are all-gathered;
      3. every segment (independent): kda_chunk_fwd from its entry state.
    When ``segment_tokens`` divides T the R segments of each sequence run as one
    batch: [B, T, H, .] is viewed, without a copy, as [B*R, T/R, H, .] and every phase
    is a single call over all B*R segments.  Otherwise the segments run one after
    another.  Returns ``(out [B,T,H,dv], final_state [B,H,dk,dv], entry_states
    [R+1,B,H,dk,dv])``."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    seg = int(segment_tokens)
    if seg <= 0:
        raise ValueError("segment_tokens must be positive")
    if T % seg == 0:
        R = T // seg

        def view(x):
            return x.reshape(B * R, seg, *x.shape[2:])

        sq, sk, sv, sg, sb = (view(x) for x in (q, k, v, g, beta))
        # phase 1: exit states from zero entry states and transitions, all segments at once
        _, exits = kda_chunk_fwd(sq, sk, sv, sg, sb, scale, None)
        trans = kda_chunk_transition(sq, sk, sg, sb)
        # [B*R, ...] in (b, r) order -> [R, B, ...] for the composition
        tr = trans.reshape(B, R, H, dk, dk).transpose(0, 1).contiguous()
        ex = exits.reshape(B, R, H, dk, dv).transpose(0, 1).contiguous()
        entry = kda_state_compose(tr, ex, initial_state)                     # phase 2
        s0 = entry[:R].transpose(0, 1).reshape(B * R, H, dk, dv).contiguous()
        out = torch.empty((B, T, H, dv), dtype=v.dtype, device=v.device)
        kda_chunk_fwd(sq, sk, sv, sg, sb, scale, s0, output_final_state=False,
                      out=out.reshape(B * R, seg, H, dv))                      # phase 3
        return out, entry[R], entry
    bounds = [(t0, min(T, t0 + seg)) for t0 in range(0, T, seg)]
    R = len(bounds)

    def piece(x, t0, t1):
        return x[:, t0:t1].contiguous()

    parts = [{n: piece(x, t0, t1) for n, x in (("q", q), ("k", k), ("v", v), ("g", g),
                                                 ("beta", beta))} for t0, t1 in bounds]
    trans = torch.empty((R, B, H, dk, dk), dtype=torch.float32, device=q.device)
    exits = torch.empty((R, B, H, dk, dv), dtype=torch.float32, device=q.device)
    for r, p in enumerate(parts):                                  # phase 1
        kda_chunk_fwd(p["q"], p["k"], p["v"], p["g"], p["beta"], scale, None,
                      final_state=exits[r])
        kda_chunk_transition(p["q"], p["k"], p["g"], p["beta"], transition=trans[r])
    entry = kda_state_compose(trans, exits, initial_state)         # phase 2
    out = torch.empty((B, T, H, dv), dtype=v.dtype, device=v.device)
    for r, ((t0, t1), p) in enumerate(zip(bounds, parts)):         # phase 3
        o, _ = kda_chunk_fwd(p["q"], p["k"], p["v"], p["g"], p["beta"], scale, entry[r],
                             output_final_state=False)
        out[:, t0:t1] = o
    return out, entry[R], entry


# short aliases
chunk_fwd = kda_chunk_fwd
chunk_fwd_varlen = kda_chunk_fwd_varlen
chunk_fwd_snapshots = kda_chunk_fwd_snapshots
chunk_fwd_prologue = kda_chunk_fwd_prologue
decode_step = kda_decode_step
chunk_bwd = kda_chunk_bwd
chunk_transition = kda_chunk_transition
state_compose = kda_state_compose
