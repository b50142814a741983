"""Kimi Delta Attention (KDA) forward and backward on AMD MI355X (gfx950).

A thin ctypes binding over the C ABI of ``libkda.so`` (declared in
include/kda.h). It only marshals arguments: checks tensor shapes, dtypes,
devices and contiguity, allocates outputs with torch, and passes raw device
pointers plus torch's current HIP stream. Every step of the computation runs
in the library's HIP kernels; there is no fallback path. If the library is
not built, calls raise ``RuntimeError``.

    o, final_state = chunk_fwd(q, k, v, g, beta, initial_state=None,
                               cu_seqlens=None, chunk_size=0, scale=1.0,
                               output_final_state=True)
    dq, dk, dv, dg, dbeta, d_initial = chunk_bwd(q, k, v, g, beta, d_o, initial_state=None,
                                                 d_final_state=None, cu_seqlens=None, scale=1.0)
    o = recurrent_step(q, k, v, g, beta, state_cache, state_slots=None, scale=1.0)
    device_check()      # raises KDAError if a kernel's bounded wait gave up since the last check
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "kda.h")

KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_HIP, KDA_ERR_DEVICE = 0, 1, 2, 3, 4
KDA_F32, KDA_BF16 = 0, 1
_DTYPES = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}


class KDAError(RuntimeError):
    """A non-OK status returned by libkda.so."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libkda.so and declare its entry points (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    P, I32, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    lib.kda_chunk_fwd.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, F,
                                  ctypes.c_int, P, P, P]
    lib.kda_chunk_fwd.restype = ctypes.c_int
    lib.kda_chunk_fwd_prologue.argtypes = [P, P, P, P, P, P, P, F, F, P, P, I32, I32, I32, I32, I32, I32,
                                           I32, F, ctypes.c_int, P, P, P]
    lib.kda_chunk_fwd_prologue.restype = ctypes.c_int
    lib.kda_prologue.argtypes = [P, P, P, P, P, P, F, F, I32, I32, I32, I32, ctypes.c_int, P, P, P, P, P]
    lib.kda_prologue.restype = ctypes.c_int
    lib.kda_recurrent_step.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I32, I32, F,
                                       ctypes.c_int, P, P]
    lib.kda_recurrent_step.restype = ctypes.c_int
    lib.kda_recurrent_step_prologue.argtypes = [P, P, P, P, P, P, P, F, F, P, P, I32, I32, I32, I32, I32, F,
                                                ctypes.c_int, P, P]
    lib.kda_recurrent_step_prologue.restype = ctypes.c_int
    lib.kda_recurrent_step_conv.argtypes = [P, P, P, P, P, P, P, P, P, I32, P, P, P, P, F, F, P, P, I32, I32, I32,
                                            I32, I32, F, ctypes.c_int, P, P]
    lib.kda_recurrent_step_conv.restype = ctypes.c_int
    lib.kda_short_conv.argtypes = [P, P, P, P, I32, I32, I32, I32, I32, ctypes.c_int, P, P, P]
    lib.kda_short_conv.restype = ctypes.c_int
    lib.kda_short_conv_bwd_workspace_bytes.argtypes = [I32, I32, I32]
    lib.kda_short_conv_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_short_conv_bwd.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32, I32, ctypes.c_int, P, ctypes.c_size_t,
                                       P, P, P, P]
    lib.kda_short_conv_bwd.restype = ctypes.c_int
    lib.kda_short_conv_step.argtypes = [P, P, P, P, I32, I32, I32, I32, ctypes.c_int, P, P]
    lib.kda_short_conv_step.restype = ctypes.c_int
    lib.kda_chunk_fwd_conv_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, ctypes.c_int, F]
    lib.kda_chunk_fwd_conv_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_chunk_fwd_conv.argtypes = [P, P, P, P, P, P, P, P, P, I32, P, P, P, P, F, F, P, P, I32, I32, I32, I32,
                                       I32, I32, I32, F, ctypes.c_int, P, ctypes.c_size_t, P, P, P, P, P, P]
    lib.kda_chunk_fwd_conv.restype = ctypes.c_int
    lib.kda_chunk_fwd_split_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32, ctypes.c_int, I32]
    lib.kda_chunk_fwd_split_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_chunk_fwd_split.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, F, ctypes.c_int,
                                        I32, P, ctypes.c_size_t, P, P, P]
    lib.kda_chunk_fwd_split.restype = ctypes.c_int
    lib.kda_chunk_fwd_split_prologue.argtypes = [P, P, P, P, P, P, P, F, F, P, P, I32, I32, I32, I32, I32, I32, I32,
                                                 F, ctypes.c_int, I32, P, ctypes.c_size_t, P, P, P]
    lib.kda_chunk_fwd_split_prologue.restype = ctypes.c_int
    lib.kda_chunk_fwd_split_static.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, F,
                                               ctypes.c_int, I32, P, P, P]
    lib.kda_chunk_fwd_split_static.restype = ctypes.c_int
    lib.kda_chunk_bwd_prologue_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32, I32]
    lib.kda_chunk_bwd_prologue_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_chunk_bwd_prologue.argtypes = [P, P, P, P, P, P, P, F, F, P, P, P, P, I32, I32, I32, I32, I32, I32, F,
                                           ctypes.c_int, P, ctypes.c_size_t, P, P, P, P, P, P, P, P, P]
    lib.kda_chunk_bwd_prologue.restype = ctypes.c_int
    lib.kda_chunk_bwd_conv_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32, I32, ctypes.c_int]
    lib.kda_chunk_bwd_conv_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_chunk_bwd_conv.argtypes = ([P] * 9 + [I32] + [P] * 4 + [F, F] + [P] * 7 + [I32] * 6 + [F, ctypes.c_int, P,
                                       ctypes.c_size_t] + [P] * 14 + [P])
    lib.kda_chunk_bwd_conv.restype = ctypes.c_int
    lib.kda_chunk_bwd_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32, I32]
    lib.kda_chunk_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_chunk_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, F, ctypes.c_int,
                                  P, ctypes.c_size_t, P, P, P, P, P, P, P]
    lib.kda_chunk_bwd.restype = ctypes.c_int
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_last_error_message.argtypes = []
    lib.kda_last_error_message.restype = ctypes.c_char_p
    lib.kda_device_check.argtypes = [P]
    lib.kda_device_check.restype = ctypes.c_int
    lib.kda_set_wait_limit.argtypes = [I32]
    lib.kda_set_wait_limit.restype = ctypes.c_int
    _lib = lib
    return lib


def declared_symbols(header: str = HEADER_PATH):
    """Names of the functions include/kda.h declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def _check(status: int):
    if status != KDA_OK:
        lib = load_library()
        msg = lib.kda_last_error_message().decode()
        name = lib.kda_status_string(status).decode()
        raise KDAError(status, f"{name}: {msg}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _chunk_outputs(B, T, H, Dk, Dv, N, dt, dev, out, final_state, output_final_state):
    if out is None:
        out = torch.empty((B, T, H, Dv), dtype=dt, device=dev)
    else:
        _need(out, "out", (B, T, H, Dv), dt, dev)
    if output_final_state:
        if final_state is None:
            final_state = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev)
        else:
            _need(final_state, "final_state", (N, H, Dk, Dv), torch.float32, dev)
    else:
        final_state = None
    return out, final_state


def _chunk_inputs(q, k, v, g, beta, initial_state, cu_seqlens, names):
    if q.dim() != 4:
        raise ValueError(f"{names[0]} must be [B,T,H,Dk]")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    dt = q.dtype
    _need(q, names[0], (B, T, H, Dk), dt, dev)
    _need(k, names[1], (B, T, H, Dk), dt, dev)
    _need(g, names[3], (B, T, H, Dk), dt, dev)
    _need(v, names[2], (B, T, H, Dv), dt, dev)
    _need(beta, names[4], (B, T, H), dt, dev)
    if cu_seqlens is not None:
        if cu_seqlens.dim() != 1:
            raise ValueError("cu_seqlens must be 1-D")
        N = cu_seqlens.numel() - 1
        _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    else:
        N = B
    if initial_state is not None:
        _need(initial_state, "initial_state", (N, H, Dk, Dv), torch.float32, dev)
    return B, T, H, Dk, Dv, N, dt, dev


def chunk_fwd(q, k, v, g, beta, initial_state=None, cu_seqlens=None, chunk_size=0, scale=1.0,
              output_final_state=True, out=None, final_state=None):
    """KDA forward over whole sequences (kda_chunk_fwd).

    q, k, g [B,T,H,Dk]; v [B,T,H,Dv]; beta [B,T,H] (all float32 or all bfloat16,
    on one GPU); initial_state [N,H,Dk,Dv] float32 or None; cu_seqlens int32
    [N+1] (B must be 1) or None (N = B). Returns (o [B,T,H,Dv], final_state
    [N,H,Dk,Dv] float32 or None).
    """
    lib = load_library()
    B, T, H, Dk, Dv, N, dt, dev = _chunk_inputs(q, k, v, g, beta, initial_state, cu_seqlens,
                                                ("q", "k", "v", "g", "beta"))
    out, final_state = _chunk_outputs(B, T, H, Dk, Dv, N, dt, dev, out, final_state, output_final_state)
    st = lib.kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                           _ptr(cu_seqlens), B, T, H, Dk, Dv, N, int(chunk_size), float(scale),
                           _DTYPES[dt], _ptr(out), _ptr(final_state), _stream(dev))
    _check(st)
    return out, final_state


def chunk_fwd_conv_workspace_bytes(B, T, H, Dk, Dv, dtype, gate_lower_bound=-5.0):
    """Bytes of workspace kda_chunk_fwd_conv needs."""
    return int(load_library().kda_chunk_fwd_conv_workspace_bytes(B, T, H, Dk, Dv, _DTYPES[dtype],
                                                                  float(gate_lower_bound)))


def chunk_fwd_conv(xq, xk, xv, wq, wk, wv, g_logit, beta_logit, A_log, dt_bias, conv_states=None, activation=True,
                   gate_lower_bound=-5.0, l2_eps=1e-6, initial_state=None, cu_seqlens=None, chunk_size=0, scale=1.0,
                   output_final_state=True, output_conv_states=True, out=None, final_state=None,
                   conv_states_out=None, workspace=None):
    """Short convolution of q, k, v then the prologue forward (kda_chunk_fwd_conv).

    xq, xk [B,T,H,Dk], xv [B,T,H,Dv] (projections before the convolution);
    wq, wk [H*Dk,4], wv [H*Dv,4] float32; conv_states: None or a triple of
    [N,3,H*D] float32 (None entries = zeros). Returns (o, final_state,
    (conv_q, conv_k, conv_v) final conv states or None)."""
    lib = load_library()
    B, T, H, Dk, Dv, N, dt, dev = _chunk_inputs(xq, xk, xv, g_logit, beta_logit, initial_state, cu_seqlens,
                                                ("xq", "xk", "xv", "g_logit", "beta_logit"))
    _need(A_log, "A_log", (Dk,), torch.float32, dev)
    _need(dt_bias, "dt_bias", (H * Dk,), torch.float32, dev)
    for w, d, name in ((wq, Dk, "wq"), (wk, Dk, "wk"), (wv, Dv, "wv")):
        _need(w, name, (H * d, 4), torch.float32, dev)
    s0 = [None, None, None] if conv_states is None else list(conv_states)
    for st, d, name in zip(s0, (Dk, Dk, Dv), ("conv_state_q", "conv_state_k", "conv_state_v")):
        if st is not None:
            _need(st, name, (N, 3, H * d), torch.float32, dev)
    out, final_state = _chunk_outputs(B, T, H, Dk, Dv, N, dt, dev, out, final_state, output_final_state)
    s1 = [None, None, None]
    if output_conv_states:
        s1 = list(conv_states_out) if conv_states_out is not None else [
            torch.empty((N, 3, H * d), dtype=torch.float32, device=dev) for d in (Dk, Dk, Dv)]
        for st, d, name in zip(s1, (Dk, Dk, Dv), ("conv_state_q_out", "conv_state_k_out", "conv_state_v_out")):
            _need(st, name, (N, 3, H * d), torch.float32, dev)
    need = chunk_fwd_conv_workspace_bytes(B, T, H, Dk, Dv, dt, gate_lower_bound)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    elif workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    st = lib.kda_chunk_fwd_conv(_ptr(xq), _ptr(xk), _ptr(xv), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(s0[0]),
                                _ptr(s0[1]), _ptr(s0[2]), int(bool(activation)), _ptr(g_logit), _ptr(beta_logit),
                                _ptr(A_log), _ptr(dt_bias), float(gate_lower_bound), float(l2_eps),
                                _ptr(initial_state), _ptr(cu_seqlens), B, T, H, Dk, Dv, N, int(chunk_size),
                                float(scale), _DTYPES[dt], _ptr(workspace), workspace.numel(), _ptr(out),
                                _ptr(final_state), _ptr(s1[0]), _ptr(s1[1]), _ptr(s1[2]), _stream(dev))
    _check(st)
    return out, final_state, (tuple(s1) if output_conv_states else None)


def chunk_fwd_split_workspace_bytes(B, T, H, Dk, Dv, N, dtype, segments):
    """Bytes of workspace kda_chunk_fwd_split needs (0 when segments <= 1)."""
    return int(load_library().kda_chunk_fwd_split_workspace_bytes(B, T, H, Dk, Dv, N, _DTYPES[dtype], segments))


def chunk_fwd_split(q, k, v, g, beta, segments, initial_state=None, cu_seqlens=None, chunk_size=0, scale=1.0,
                    output_final_state=True, out=None, final_state=None, workspace=None):
    """``chunk_fwd`` with every sequence cut into ``segments`` pieces run in
    parallel and joined by the affine form of the state map
    (kda_chunk_fwd_split). ``workspace``: a uint8 device tensor of at least
    ``chunk_fwd_split_workspace_bytes`` bytes, or None to allocate one."""
    lib = load_library()
    B, T, H, Dk, Dv, N, dt, dev = _chunk_inputs(q, k, v, g, beta, initial_state, cu_seqlens,
                                                ("q", "k", "v", "g", "beta"))
    out, final_state = _chunk_outputs(B, T, H, Dk, Dv, N, dt, dev, out, final_state, output_final_state)
    need = chunk_fwd_split_workspace_bytes(B, T, H, Dk, Dv, N, dt, int(segments))
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    elif workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    st = lib.kda_chunk_fwd_split(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                                 _ptr(cu_seqlens), B, T, H, Dk, Dv, N, int(chunk_size), float(scale), _DTYPES[dt],
                                 int(segments), _ptr(workspace), workspace.numel(), _ptr(out), _ptr(final_state),
                                 _stream(dev))
    _check(st)
    return out, final_state


SPLIT_STATIC_SCRATCH_BYTES = 128 << 20   # KDA_SPLIT_STATIC_SCRATCH_BYTES


def chunk_fwd_split_prologue(q_raw, k_raw, v, g_logit, beta_logit, A_log, dt_bias, segments, gate_lower_bound=-5.0,
                             l2_eps=1e-6, initial_state=None, cu_seqlens=None, chunk_size=0, scale=1.0,
                             output_final_state=True, out=None, final_state=None, workspace=None):
    """``chunk_fwd_split`` from raw projections (kda_chunk_fwd_split_prologue):
    inputs as ``chunk_fwd_prologue``, ``segments`` and ``workspace`` as
    ``chunk_fwd_split``. Returns (o, final_state or None)."""
    lib = load_library()
    B, T, H, Dk, Dv, N, dt, dev = _chunk_inputs(q_raw, k_raw, v, g_logit, beta_logit, initial_state, cu_seqlens,
                                                ("q_raw", "k_raw", "v", "g_logit", "beta_logit"))
    _need(A_log, "A_log", (Dk,), torch.float32, dev)
    _need(dt_bias, "dt_bias", (H * Dk,), torch.float32, dev)
    out, final_state = _chunk_outputs(B, T, H, Dk, Dv, N, dt, dev, out, final_state, output_final_state)
    need = chunk_fwd_split_workspace_bytes(B, T, H, Dk, Dv, N, dt, segments)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    elif workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    st = lib.kda_chunk_fwd_split_prologue(_ptr(q_raw), _ptr(k_raw), _ptr(v), _ptr(g_logit), _ptr(beta_logit),
                                          _ptr(A_log), _ptr(dt_bias), float(gate_lower_bound), float(l2_eps),
                                          _ptr(initial_state), _ptr(cu_seqlens), B, T, H, Dk, Dv, N, int(chunk_size),
                                          float(scale), _DTYPES[dt], int(segments), _ptr(workspace),
                                          workspace.numel(), _ptr(out), _ptr(final_state), _stream(dev))
    _check(st)
    return out, final_state


def chunk_fwd_split_static(q, k, v, g, beta, segments, initial_state=None, cu_seqlens=None, chunk_size=0,
                           scale=1.0, output_final_state=True, out=None, final_state=None):
    """``chunk_fwd_split`` on the library's static scratch instead of a
    workspace (kda_chunk_fwd_split_static): with ``out`` (and ``final_state``)
    passed in, nothing is allocated. Sizes whose workspace exceeds
    SPLIT_STATIC_SCRATCH_BYTES are refused; overlapping calls on one device
    race on the scratch."""
    lib = load_library()
    B, T, H, Dk, Dv, N, dt, dev = _chunk_inputs(q, k, v, g, beta, initial_state, cu_seqlens,
                                                ("q", "k", "v", "g", "beta"))
    out, final_state = _chunk_outputs(B, T, H, Dk, Dv, N, dt, dev, out, final_state, output_final_state)
    st = lib.kda_chunk_fwd_split_static(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                                        _ptr(cu_seqlens), B, T, H, Dk, Dv, N, int(chunk_size), float(scale),
                                        _DTYPES[dt], int(segments), _ptr(out), _ptr(final_state), _stream(dev))
    _check(st)
    return out, final_state


def chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, N, packed):
    """Bytes of workspace kda_chunk_bwd needs (kda_chunk_bwd_workspace_bytes)."""
    return int(load_library().kda_chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, N, int(bool(packed))))


def chunk_bwd(q, k, v, g, beta, d_o, initial_state=None, d_final_state=None, cu_seqlens=None, scale=1.0,
              workspace=None, want_d_initial=True):
    """Gradients of <d_o, o> + <d_final_state, final_state> for ``chunk_fwd`` (kda_chunk_bwd).

    Inputs as for ``chunk_fwd``; d_o [B,T,H,Dv] in the inputs' dtype;
    d_final_state [N,H,Dk,Dv] float32 or None. ``workspace`` is a uint8 device
    tensor of at least ``chunk_bwd_workspace_bytes`` bytes, or None to
    allocate one. Returns float32 (dq, dk, dv, dg, dbeta, d_initial_state or
    None).
    """
    lib = load_library()
    B, T, H, Dk, Dv, N, dt, dev = _chunk_inputs(q, k, v, g, beta, initial_state, cu_seqlens,
                                                ("q", "k", "v", "g", "beta"))
    _need(d_o, "d_o", (B, T, H, Dv), dt, dev)
    if d_final_state is not None:
        _need(d_final_state, "d_final_state", (N, H, Dk, Dv), torch.float32, dev)
    need = chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, N, cu_seqlens is not None)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    elif workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    f32 = dict(dtype=torch.float32, device=dev)
    dq = torch.empty((B, T, H, Dk), **f32)
    dk = torch.empty((B, T, H, Dk), **f32)
    dg = torch.empty((B, T, H, Dk), **f32)
    dv = torch.empty((B, T, H, Dv), **f32)
    dbeta = torch.empty((B, T, H), **f32)
    d_init = torch.empty((N, H, Dk, Dv), **f32) if want_d_initial else None
    st = lib.kda_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                           _ptr(cu_seqlens), _ptr(d_o), _ptr(d_final_state), B, T, H, Dk, Dv, N, float(scale),
                           _DTYPES[dt], _ptr(workspace), workspace.numel(), _ptr(dq), _ptr(dk), _ptr(dv),
                           _ptr(dg), _ptr(dbeta), _ptr(d_init), _stream(dev))
    _check(st)
    return dq, dk, dv, dg, dbeta, d_init


def chunk_bwd_prologue_workspace_bytes(B, T, H, Dk, Dv, N, packed):
    """Bytes of workspace kda_chunk_bwd_prologue needs."""
    return int(load_library().kda_chunk_bwd_prologue_workspace_bytes(B, T, H, Dk, Dv, N, int(bool(packed))))


def chunk_bwd_prologue(q_raw, k_raw, v, g_logit, beta_logit, A_log, dt_bias, d_o, gate_lower_bound=-5.0,
                       l2_eps=1e-6, initial_state=None, d_final_state=None, cu_seqlens=None, scale=1.0,
                       workspace=None, want_d_initial=True):
    """Gradients for ``chunk_fwd_prologue`` (kda_chunk_bwd_prologue): returns
    float32 (dq_raw, dk_raw, dv, dg_logit, dbeta_logit, dA_log, ddt_bias,
    d_initial_state or None)."""
    lib = load_library()
    B, T, H, Dk, Dv, N, dt, dev = _chunk_inputs(q_raw, k_raw, v, g_logit, beta_logit, initial_state, cu_seqlens,
                                                ("q_raw", "k_raw", "v", "g_logit", "beta_logit"))
    _need(A_log, "A_log", (Dk,), torch.float32, dev)
    _need(dt_bias, "dt_bias", (H * Dk,), torch.float32, dev)
    _need(d_o, "d_o", (B, T, H, Dv), dt, dev)
    if d_final_state is not None:
        _need(d_final_state, "d_final_state", (N, H, Dk, Dv), torch.float32, dev)
    need = chunk_bwd_prologue_workspace_bytes(B, T, H, Dk, Dv, N, cu_seqlens is not None)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    elif workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    f32 = dict(dtype=torch.float32, device=dev)
    dq = torch.empty((B, T, H, Dk), **f32)
    dk = torch.empty((B, T, H, Dk), **f32)
    dg = torch.empty((B, T, H, Dk), **f32)
    dv = torch.empty((B, T, H, Dv), **f32)
    dbeta = torch.empty((B, T, H), **f32)
    dA = torch.empty((Dk,), **f32)
    dbias = torch.empty((H * Dk,), **f32)
    d_init = torch.empty((N, H, Dk, Dv), **f32) if want_d_initial else None
    st = lib.kda_chunk_bwd_prologue(_ptr(q_raw), _ptr(k_raw), _ptr(v), _ptr(g_logit), _ptr(beta_logit), _ptr(A_log),
                                    _ptr(dt_bias), float(gate_lower_bound), float(l2_eps), _ptr(initial_state),
                                    _ptr(cu_seqlens), _ptr(d_o), _ptr(d_final_state), B, T, H, Dk, Dv, N,
                                    float(scale), _DTYPES[dt], _ptr(workspace), workspace.numel(), _ptr(dq),
                                    _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dA), _ptr(dbias), _ptr(d_init),
                                    _stream(dev))
    _check(st)
    return dq, dk, dv, dg, dbeta, dA, dbias, d_init


def chunk_bwd_conv_workspace_bytes(B, T, H, Dk, Dv, N, packed, dtype):
    """Bytes of workspace kda_chunk_bwd_conv needs."""
    return int(load_library().kda_chunk_bwd_conv_workspace_bytes(B, T, H, Dk, Dv, N, int(bool(packed)),
                                                                  _DTYPES[dtype]))


def chunk_bwd_conv(xq, xk, xv, wq, wk, wv, g_logit, beta_logit, A_log, dt_bias, d_o, conv_states=None,
                   d_conv_final=None, activation=True, gate_lower_bound=-5.0, l2_eps=1e-6, initial_state=None,
                   d_final_state=None, cu_seqlens=None, scale=1.0, workspace=None, want_d_initial=True,
                   want_d_conv_states=True):
    """Gradients for ``chunk_fwd_conv`` (kda_chunk_bwd_conv). conv_states and
    d_conv_final: None or a triple (q, k, v) of [N,3,H*D] float32 (None
    entries = zeros). Returns a dict of float32 gradients keyed xq, xk, xv
    ([B,T,H,D]), wq, wk, wv ([H*D,4]), conv_state_q, conv_state_k,
    conv_state_v ([N,3,H*D] or None), g_logit, beta_logit, A_log, dt_bias,
    initial_state (or None)."""
    lib = load_library()
    B, T, H, Dk, Dv, N, dt, dev = _chunk_inputs(xq, xk, xv, g_logit, beta_logit, initial_state, cu_seqlens,
                                                ("xq", "xk", "xv", "g_logit", "beta_logit"))
    _need(A_log, "A_log", (Dk,), torch.float32, dev)
    _need(dt_bias, "dt_bias", (H * Dk,), torch.float32, dev)
    _need(d_o, "d_o", (B, T, H, Dv), dt, dev)
    if d_final_state is not None:
        _need(d_final_state, "d_final_state", (N, H, Dk, Dv), torch.float32, dev)
    Ds = (Dk, Dk, Dv)
    for w, d, name in zip((wq, wk, wv), Ds, ("wq", "wk", "wv")):
        _need(w, name, (H * d, 4), torch.float32, dev)
    s0 = [None, None, None] if conv_states is None else list(conv_states)
    dfin = [None, None, None] if d_conv_final is None else list(d_conv_final)
    for lst, what in ((s0, "conv_state"), (dfin, "d_conv_final")):
        for st_, d, j in zip(lst, Ds, "qkv"):
            if st_ is not None:
                _need(st_, f"{what}_{j}", (N, 3, H * d), torch.float32, dev)
    need = chunk_bwd_conv_workspace_bytes(B, T, H, Dk, Dv, N, cu_seqlens is not None, dt)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    elif workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    f32 = dict(dtype=torch.float32, device=dev)
    g = {"xq": torch.empty((B, T, H, Dk), **f32), "xk": torch.empty((B, T, H, Dk), **f32),
         "xv": torch.empty((B, T, H, Dv), **f32)}
    for j, d in zip("qkv", Ds):
        g["w" + j] = torch.empty((H * d, 4), **f32)
        g["conv_state_" + j] = torch.empty((N, 3, H * d), **f32) if want_d_conv_states else None
    g["g_logit"] = torch.empty((B, T, H, Dk), **f32)
    g["beta_logit"] = torch.empty((B, T, H), **f32)
    g["A_log"] = torch.empty((Dk,), **f32)
    g["dt_bias"] = torch.empty((H * Dk,), **f32)
    g["initial_state"] = torch.empty((N, H, Dk, Dv), **f32) if want_d_initial else None
    st = lib.kda_chunk_bwd_conv(_ptr(xq), _ptr(xk), _ptr(xv), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(s0[0]),
                                _ptr(s0[1]), _ptr(s0[2]), int(bool(activation)), _ptr(g_logit), _ptr(beta_logit),
                                _ptr(A_log), _ptr(dt_bias), float(gate_lower_bound), float(l2_eps),
                                _ptr(initial_state), _ptr(cu_seqlens), _ptr(d_o), _ptr(d_final_state),
                                _ptr(dfin[0]), _ptr(dfin[1]), _ptr(dfin[2]), B, T, H, Dk, Dv, N, float(scale),
                                _DTYPES[dt], _ptr(workspace), workspace.numel(), _ptr(g["xq"]), _ptr(g["xk"]),
                                _ptr(g["xv"]), _ptr(g["wq"]), _ptr(g["wk"]), _ptr(g["wv"]), _ptr(g["conv_state_q"]),
                                _ptr(g["conv_state_k"]), _ptr(g["conv_state_v"]), _ptr(g["g_logit"]),
                                _ptr(g["beta_logit"]), _ptr(g["A_log"]), _ptr(g["dt_bias"]),
                                _ptr(g["initial_state"]), _stream(dev))
    _check(st)
    return g


def chunk_fwd_prologue(q_raw, k_raw, v, g_logit, beta_logit, A_log, dt_bias, gate_lower_bound=-5.0,
                       l2_eps=1e-6, initial_state=None, cu_seqlens=None, chunk_size=0, scale=1.0,
                       output_final_state=True, out=None, final_state=None):
    """KDA forward from the raw projections with the gate, beta and L2-norm
    prologue inside the chunk kernel (kda_chunk_fwd_prologue).

    q_raw, k_raw, g_logit [B,T,H,Dk]; v [B,T,H,Dv]; beta_logit [B,T,H] (one
    dtype, float32 or bfloat16); A_log [Dk] and dt_bias [H*Dk] float32 on the
    same GPU. Other arguments and the return value as ``chunk_fwd``.
    """
    lib = load_library()
    B, T, H, Dk, Dv, N, dt, dev = _chunk_inputs(q_raw, k_raw, v, g_logit, beta_logit, initial_state,
                                                cu_seqlens, ("q_raw", "k_raw", "v", "g_logit", "beta_logit"))
    _need(A_log, "A_log", (Dk,), torch.float32, dev)
    _need(dt_bias, "dt_bias", (H * Dk,), torch.float32, dev)
    out, final_state = _chunk_outputs(B, T, H, Dk, Dv, N, dt, dev, out, final_state, output_final_state)
    st = lib.kda_chunk_fwd_prologue(_ptr(q_raw), _ptr(k_raw), _ptr(v), _ptr(g_logit), _ptr(beta_logit),
                                    _ptr(A_log), _ptr(dt_bias), float(gate_lower_bound), float(l2_eps),
                                    _ptr(initial_state), _ptr(cu_seqlens), B, T, H, Dk, Dv, N,
                                    int(chunk_size), float(scale), _DTYPES[dt], _ptr(out), _ptr(final_state),
                                    _stream(dev))
    _check(st)
    return out, final_state


def prologue(q_raw, k_raw, g_logit, beta_logit, A_log, dt_bias, gate_lower_bound=-5.0, l2_eps=1e-6, out=None):
    """The gate, beta and normalisation prologue alone (kda_prologue): q_raw,
    k_raw, g_logit [B,T,H,Dk] and beta_logit [B,T,H] (one dtype); A_log [Dk],
    dt_bias [H*Dk] float32. Returns (q, k, g, beta) in the input dtype; ``out``
    may give the four output tensors (each may be its own input)."""
    lib = load_library()
    if q_raw.dim() != 4:
        raise ValueError("q_raw must be [B,T,H,Dk]")
    B, T, H, Dk = q_raw.shape
    dev, dt = q_raw.device, q_raw.dtype
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}")
    for t, n, shp in ((q_raw, "q_raw", (B, T, H, Dk)), (k_raw, "k_raw", (B, T, H, Dk)),
                      (g_logit, "g_logit", (B, T, H, Dk)), (beta_logit, "beta_logit", (B, T, H))):
        _need(t, n, shp, dt, dev)
    _need(A_log, "A_log", (Dk,), torch.float32, dev)
    _need(dt_bias, "dt_bias", (H * Dk,), torch.float32, dev)
    if out is None:
        out = (torch.empty_like(q_raw), torch.empty_like(k_raw), torch.empty_like(g_logit),
               torch.empty_like(beta_logit))
    for t, n, shp in zip(out, ("q", "k", "g", "beta"), ((B, T, H, Dk),) * 3 + ((B, T, H),)):
        _need(t, n, shp, dt, dev)
    st = lib.kda_prologue(_ptr(q_raw), _ptr(k_raw), _ptr(g_logit), _ptr(beta_logit), _ptr(A_log), _ptr(dt_bias),
                          float(gate_lower_bound), float(l2_eps), B, T, H, Dk, _DTYPES[dt], *(_ptr(t) for t in out),
                          _stream(dev))
    _check(st)
    return tuple(out)


def short_conv(x, weight, conv_state=None, cu_seqlens=None, activation=True, output_final_state=True,
               out=None, final_state=None):
    """Short causal depthwise convolution (kernel 4) over time (kda_short_conv).

    x [B,T,C] or [B,T,H,D] (float32 or bfloat16; C = H*D); weight [C,4]
    float32; conv_state [N,3,C] float32 or None (zeros); cu_seqlens int32
    [N+1] (B must be 1) or None. Returns (y like x, final conv state [N,3,C]
    float32 or None).
    """
    lib = load_library()
    if x.dim() not in (3, 4):
        raise ValueError("x must be [B,T,C] or [B,T,H,D]")
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    if x.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {x.dtype}")
    B, T = x.shape[0], x.shape[1]
    C = x[0, 0].numel() if T > 0 else int(torch.tensor(x.shape[2:]).prod())
    _need(x, "x", tuple(x.shape), x.dtype, dev)
    _need(weight, "weight", (C, 4), torch.float32, dev)
    if cu_seqlens is not None:
        N = cu_seqlens.numel() - 1
        _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    else:
        N = B
    if conv_state is not None:
        _need(conv_state, "conv_state", (N, 3, C), torch.float32, dev)
    if out is None:
        out = torch.empty_like(x)
    else:
        _need(out, "out", tuple(x.shape), x.dtype, dev)
    if output_final_state:
        if final_state is None:
            final_state = torch.empty((N, 3, C), dtype=torch.float32, device=dev)
        else:
            _need(final_state, "final_state", (N, 3, C), torch.float32, dev)
    else:
        final_state = None
    st = lib.kda_short_conv(_ptr(x), _ptr(weight), _ptr(conv_state), _ptr(cu_seqlens), B, T, C, N,
                            int(bool(activation)), _DTYPES[x.dtype], _ptr(out), _ptr(final_state), _stream(dev))
    _check(st)
    return out, final_state


def short_conv_bwd_workspace_bytes(B, T, C):
    """Device workspace bytes kda_short_conv_bwd needs (kda_short_conv_bwd_workspace_bytes)."""
    return int(load_library().kda_short_conv_bwd_workspace_bytes(B, T, C))


def short_conv_bwd(x, weight, dy, conv_state=None, d_final_state=None, cu_seqlens=None, activation=True,
                   want_d_state=True, workspace=None, out=None):
    """Gradients for ``short_conv`` (kda_short_conv_bwd): dy float32 [B,T,C]
    (x may be [B,T,C] or [B,T,H,D]); returns float32 (dx [B,T,C],
    dweight [C,4], d_state [N,3,C] or None). ``out`` may supply dx."""
    lib = load_library()
    if x.dim() == 4:
        x = x.reshape(x.shape[0], x.shape[1], -1)
    B, T, C = x.shape
    dev = x.device
    if x.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {x.dtype}")
    _need(x, "x", (B, T, C), x.dtype, dev)
    _need(weight, "weight", (C, 4), torch.float32, dev)
    dy = dy.reshape(B, T, C)
    _need(dy, "dy", (B, T, C), torch.float32, dev)
    if cu_seqlens is not None:
        N = cu_seqlens.numel() - 1
        _need(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    else:
        N = B
    if conv_state is not None:
        _need(conv_state, "conv_state", (N, 3, C), torch.float32, dev)
    if d_final_state is not None:
        _need(d_final_state, "d_final_state", (N, 3, C), torch.float32, dev)
    need = int(lib.kda_short_conv_bwd_workspace_bytes(B, T, C))
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    elif workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    if out is None:
        out = torch.empty((B, T, C), dtype=torch.float32, device=dev)
    _need(out, "out", (B, T, C), torch.float32, dev)
    dx = out
    dw = torch.empty((C, 4), dtype=torch.float32, device=dev)
    dst = torch.empty((N, 3, C), dtype=torch.float32, device=dev) if want_d_state else None
    st = lib.kda_short_conv_bwd(_ptr(x), _ptr(weight), _ptr(conv_state), _ptr(cu_seqlens), _ptr(dy),
                                _ptr(d_final_state), B, T, C, N, int(bool(activation)), _DTYPES[x.dtype],
                                _ptr(workspace), workspace.numel(), _ptr(dx), _ptr(dw), _ptr(dst), _stream(dev))
    _check(st)
    return dx, dw, dst


def short_conv_step(x, weight, conv_cache, cache_slots=None, activation=True, out=None):
    """One decode step of the short convolution (kda_short_conv_step).

    x [Nb,C] or [Nb,H,D]; weight [C,4] float32; conv_cache [n_slots,3,C]
    float32 (updated in place); cache_slots int32 [Nb] or None. Returns y like x.
    """
    lib = load_library()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    if x.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {x.dtype}")
    Nb = x.shape[0]
    C = conv_cache.shape[-1]
    _need(x, "x", tuple(x.shape), x.dtype, dev)
    if x[0].numel() != C if Nb > 0 else False:
        raise ValueError("x's channels must match conv_cache")
    _need(weight, "weight", (C, 4), torch.float32, dev)
    _need(conv_cache, "conv_cache", (conv_cache.shape[0], 3, C), torch.float32, dev)
    if cache_slots is not None:
        _need(cache_slots, "cache_slots", (Nb,), torch.int32, dev)
    if out is None:
        out = torch.empty_like(x)
    else:
        _need(out, "out", tuple(x.shape), x.dtype, dev)
    st = lib.kda_short_conv_step(_ptr(x), _ptr(weight), _ptr(conv_cache), _ptr(cache_slots), conv_cache.shape[0],
                                 Nb, C, int(bool(activation)), _DTYPES[x.dtype], _ptr(out), _stream(dev))
    _check(st)
    return out


def recurrent_step(q, k, v, g, beta, state_cache, state_slots=None, scale=1.0, out=None):
    """One KDA decode step against ``state_cache`` (updated in place; kda_recurrent_step).

    q, k, g [Nb,H,Dk]; v [Nb,H,Dv]; beta [Nb,H]; state_cache [n_slots,H,Dk,Dv]
    float32; state_slots int32 [Nb] (distinct) or None (row r -> slot r).
    Returns o [Nb,H,Dv].
    """
    lib = load_library()
    if q.dim() != 3:
        raise ValueError("q must be [Nb,H,Dk]")
    Nb, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    dt = q.dtype
    _need(q, "q", (Nb, H, Dk), dt, dev)
    _need(k, "k", (Nb, H, Dk), dt, dev)
    _need(g, "g", (Nb, H, Dk), dt, dev)
    _need(v, "v", (Nb, H, Dv), dt, dev)
    _need(beta, "beta", (Nb, H), dt, dev)
    if state_cache.dim() != 4:
        raise ValueError("state_cache must be [n_slots,H,Dk,Dv]")
    n_slots = state_cache.shape[0]
    _need(state_cache, "state_cache", (n_slots, H, Dk, Dv), torch.float32, dev)
    if state_slots is not None:
        _need(state_slots, "state_slots", (Nb,), torch.int32, dev)
    if out is None:
        out = torch.empty((Nb, H, Dv), dtype=dt, device=dev)
    else:
        _need(out, "out", (Nb, H, Dv), dt, dev)
    st = lib.kda_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_cache),
                                _ptr(state_slots), n_slots, Nb, H, Dk, Dv, float(scale),
                                _DTYPES[dt], _ptr(out), _stream(dev))
    _check(st)
    return out


def _step_shapes(q, v, state_cache, state_slots):
    if q.dim() != 3:
        raise ValueError("q must be [Nb,H,Dk]")
    Nb, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    if state_cache.dim() != 4:
        raise ValueError("state_cache must be [n_slots,H,Dk,Dv]")
    n_slots = state_cache.shape[0]
    _need(state_cache, "state_cache", (n_slots, H, Dk, Dv), torch.float32, dev)
    if state_slots is not None:
        _need(state_slots, "state_slots", (Nb,), torch.int32, dev)
    return Nb, H, Dk, Dv, n_slots, dev


def _step_raw_inputs(q, k, v, g_logit, beta_logit, A_log, dt_bias, names):
    Nb, H, Dk = q.shape
    Dv = v.shape[-1]
    dt, dev = q.dtype, q.device
    for t, n, shp in ((q, names[0], (Nb, H, Dk)), (k, names[1], (Nb, H, Dk)), (v, names[2], (Nb, H, Dv)),
                      (g_logit, "g_logit", (Nb, H, Dk)), (beta_logit, "beta_logit", (Nb, H))):
        _need(t, n, shp, dt, dev)
    _need(A_log, "A_log", (Dk,), torch.float32, dev)
    _need(dt_bias, "dt_bias", (H * Dk,), torch.float32, dev)


def recurrent_step_prologue(q_raw, k_raw, v, g_logit, beta_logit, A_log, dt_bias, state_cache, state_slots=None,
                            gate_lower_bound=-5.0, l2_eps=1e-6, scale=1.0, out=None):
    """One decode step from raw projections (kda_recurrent_step_prologue): the
    gate, beta and normalisation prologue, then the step against
    ``state_cache`` (updated in place).

    q_raw, k_raw, g_logit [Nb,H,Dk]; v [Nb,H,Dv]; beta_logit [Nb,H]; A_log [Dk]
    and dt_bias [H*Dk] float32; state_cache [n_slots,H,Dk,Dv] float32;
    state_slots int32 [Nb] or None. Returns o [Nb,H,Dv].
    """
    lib = load_library()
    Nb, H, Dk, Dv, n_slots, dev = _step_shapes(q_raw, v, state_cache, state_slots)
    _step_raw_inputs(q_raw, k_raw, v, g_logit, beta_logit, A_log, dt_bias, ("q_raw", "k_raw", "v"))
    dt = q_raw.dtype
    if out is None:
        out = torch.empty((Nb, H, Dv), dtype=dt, device=dev)
    else:
        _need(out, "out", (Nb, H, Dv), dt, dev)
    st = lib.kda_recurrent_step_prologue(_ptr(q_raw), _ptr(k_raw), _ptr(v), _ptr(g_logit), _ptr(beta_logit),
                                         _ptr(A_log), _ptr(dt_bias), float(gate_lower_bound), float(l2_eps),
                                         _ptr(state_cache), _ptr(state_slots), n_slots, Nb, H, Dk, Dv, float(scale),
                                         _DTYPES[dt], _ptr(out), _stream(dev))
    _check(st)
    return out


def recurrent_step_conv(xq, xk, xv, wq, wk, wv, conv_caches, g_logit, beta_logit, A_log, dt_bias, state_cache,
                        state_slots=None, activation=True, gate_lower_bound=-5.0, l2_eps=1e-6, scale=1.0, out=None):
    """One generated token from the projections before the short convolution
    (kda_recurrent_step_conv): the convolution step of q, k and v over
    ``conv_caches``, the prologue and the decode step, all caches updated in
    place.

    xq, xk, g_logit [Nb,H,Dk]; xv [Nb,H,Dv]; beta_logit [Nb,H]; wq, wk [H*Dk,4]
    and wv [H*Dv,4] float32; conv_caches (q, k, v) [n_slots,3,H*D] float32,
    indexed by the state slots; the rest as for ``recurrent_step_prologue``.
    Returns o [Nb,H,Dv].
    """
    lib = load_library()
    Nb, H, Dk, Dv, n_slots, dev = _step_shapes(xq, xv, state_cache, state_slots)
    _step_raw_inputs(xq, xk, xv, g_logit, beta_logit, A_log, dt_bias, ("xq", "xk", "xv"))
    cq, ck, cv = conv_caches
    for t, n, C in ((wq, "wq", H * Dk), (wk, "wk", H * Dk), (wv, "wv", H * Dv)):
        _need(t, n, (C, 4), torch.float32, dev)
    for t, n, C in ((cq, "conv_cache_q", H * Dk), (ck, "conv_cache_k", H * Dk), (cv, "conv_cache_v", H * Dv)):
        _need(t, n, (n_slots, 3, C), torch.float32, dev)
    dt = xq.dtype
    if out is None:
        out = torch.empty((Nb, H, Dv), dtype=dt, device=dev)
    else:
        _need(out, "out", (Nb, H, Dv), dt, dev)
    st = lib.kda_recurrent_step_conv(_ptr(xq), _ptr(xk), _ptr(xv), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(cq),
                                     _ptr(ck), _ptr(cv), int(bool(activation)), _ptr(g_logit), _ptr(beta_logit),
                                     _ptr(A_log), _ptr(dt_bias), float(gate_lower_bound), float(l2_eps),
                                     _ptr(state_cache), _ptr(state_slots), n_slots, Nb, H, Dk, Dv, float(scale),
                                     _DTYPES[dt], _ptr(out), _stream(dev))
    _check(st)
    return out


def device_check(device=None):
    """Wait for torch's current stream on ``device`` and raise ``KDAError``
    (status KDA_ERR_DEVICE) if a bounded wait of any library kernel on that
    device gave up since the previous check."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    lib = load_library()
    with torch.cuda.device(dev):
        _check(lib.kda_device_check(_stream(dev)))


def set_wait_limit(polls: int):
    """Polls of one bounded wait before it gives up, for calls launched from now on."""
    _check(load_library().kda_set_wait_limit(int(polls)))
