"""Seeded synthetic inputs shaped like the Kimi K3 KDA workloads.

This module only draws and shapes random numbers; it holds none of the
recurrence's arithmetic. Both the oracle-side tests and the GPU path take their
inputs from here.

Shapes follow the pages: K3 has 96 KDA heads of head_dim 128 (hysenlabs
"kimi-k3-mlx", section "Attention is 93 layers split between KDA and a NoPE
gated MLA"); the log-decay g is per token, head and key channel, shape
(B,T,96,128) (same article, section "The A_log shape mismatch ..."); the gate
is bounded below by gate_lower_bound = -5.0 (section "Attention is 93
layers ..."); packed variable-length batches are concatenated on T with
cumulative offsets (ISEEKYAN/k3 README, packed THD with context parallelism).

Recipe (numpy PCG64 generators, float32 draws):
  streams: lengths 0, q 1, k 2, v 3, g_raw 4, beta_raw 5, S0 6. Stream s of a
  workload with seed S is cut into fixed blocks of BLOCK_ROWS leading-axis
  rows (tokens; state slots for S0); block b is drawn from
  ``default_rng([S, s, b])``. Blocks are independent, so large tensors are
  filled on several threads and the values never depend on the thread count.
  q, k  ~ N(0,1), then L2-normalised over d_k per (token, head), in float32
  v     ~ N(0,1)
  g     = -5 * sigmoid(g_raw), g_raw ~ N(0,1)   (per channel, in [-5, 0))
  beta  = sigmoid(beta_raw), beta_raw ~ N(0,1)  (per token and head)
  S0    ~ N(0, 0.02) float32 when requested (0.02 is the standard deviation)
  d_o   ~ N(0,1) (stream 9), d_final ~ N(0, 0.1) float32 (stream 10): the
        output and final-state cotangents of the backward workloads
  decode from raw projections: q_raw, k_raw, v, g_logit, beta_logit ~ N(0,1)
        per step (stream 13); gate parameters A_log, dt_bias ~ N(0, 0.5)
        (streams 7, 8); convolution taps ~ N(0, 0.5) (stream 11) and caches
        ~ N(0,1) (stream 12), per projection
then, for bf16 workloads, q,k,v,g,beta are rounded to bf16 (round to nearest
even). States stay float32.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np
import torch

K3_HEADS = 96
K3_HEAD_DIM = 128
GATE_LOWER_BOUND = -5.0


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    Dk: int
    Dv: int
    chunk: int
    dtype: str            # "f32" or "bf16"
    init_state: bool      # S0 ~ N(0, 0.02) when True, zeros otherwise
    n_seqs: int = 0       # >0: packed batch of n_seqs sequences (B == 1, T = sum of lengths)
    len_lo: int = 0
    len_hi: int = 0
    seed: int = 0


# The five workloads the method is measured on (sizes as stated for the K3 shape).
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 64, 2, 16, 16, 16, "f32", False, seed=0),
    "k3_t4096": Workload("k3_t4096", 1, 4096, K3_HEADS, 128, 128, 64, "bf16", False, seed=1),
    "k3_t32768_s0": Workload("k3_t32768_s0", 1, 32768, K3_HEADS, 128, 128, 64, "bf16", True, seed=2),
    "k3_varlen16": Workload("k3_varlen16", 1, 0, K3_HEADS, 128, 128, 64, "bf16", False,
                            n_seqs=16, len_lo=128, len_hi=8192, seed=3),
}
DECODE = dict(name="k3_decode_b256", Nb=256, H=K3_HEADS, Dk=128, Dv=128, steps=128, seed=4)


def _sigmoid(x):
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _l2norm(x):
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-6))).astype(np.float32)


def _round(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def packed_lengths(rng, n, lo, hi):
    """n integer lengths uniform on [lo, hi], both ends included."""
    return rng.integers(lo, hi + 1, size=n)


BLOCK_ROWS = 1024
_STREAM = dict(lengths=0, q=1, k=2, v=3, g=4, beta=5, s0=6, A_log=7, dt_bias=8, d_o=9, d_final=10, conv_w=11,
               conv_cache=12, decode_raw=13)


def _pool_size():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _blocked(seed, stream, shape, finish):
    """float32 array of ``shape`` whose leading-axis blocks of BLOCK_ROWS rows
    are standard normals from default_rng([seed, stream, block]), each block
    passed through ``finish`` (an elementwise or per-row map) in place."""
    out = np.empty(shape, dtype=np.float32)
    rows = shape[0]
    nblk = (rows + BLOCK_ROWS - 1) // BLOCK_ROWS

    def fill(b):
        lo, hi = b * BLOCK_ROWS, min(rows, (b + 1) * BLOCK_ROWS)
        x = np.random.default_rng([seed, stream, b]).standard_normal((hi - lo,) + tuple(shape[1:]),
                                                                      dtype=np.float32)
        out[lo:hi] = finish(x)

    if nblk <= 1:
        for b in range(nblk):
            fill(b)
    else:
        with ThreadPoolExecutor(max_workers=_pool_size()) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def make_chunk_inputs(B, T, H, Dk, Dv, seed, dtype="bf16", init_state=False, lengths=None,
                      n_seqs=0, len_lo=0, len_hi=0, g_mode="default", beta_mode="default",
                      v_zero=False, s0_std=0.02):
    """Draw one forward workload.

    Returns a dict of CPU torch tensors: q,k,g [B,T,H,Dk], v [B,T,H,Dv], beta
    [B,T,H] in ``dtype`` ("bf16" or "f32"); initial_state [N,H,Dk,Dv] float32
    or None; cu_seqlens int32 [N+1] or None.

    Variants used by the stress tests: g_mode "weak" (-0.05*sigmoid), "zero",
    "bound" (g == -5 everywhere); beta_mode "one"; v_zero; s0_std.
    """
    cu = None
    if lengths is None and n_seqs > 0:
        lengths = packed_lengths(np.random.default_rng([seed, _STREAM["lengths"]]), n_seqs, len_lo, len_hi)
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        B, T = 1, int(cu[-1])
    N = B if cu is None else len(cu) - 1
    rows = B * T
    ident = lambda x: x  # noqa: E731
    gmap = {"default": lambda x: np.float32(GATE_LOWER_BOUND) * _sigmoid(x),
            "weak": lambda x: np.float32(-0.05) * _sigmoid(x),
            "zero": np.zeros_like,
            "bound": lambda x: np.full_like(x, GATE_LOWER_BOUND)}
    bmap = {"default": _sigmoid, "one": np.ones_like, "zero": np.zeros_like}
    if g_mode not in gmap:
        raise ValueError(g_mode)
    if beta_mode not in bmap:
        raise ValueError(beta_mode)
    q = _blocked(seed, _STREAM["q"], (rows, H, Dk), _l2norm)
    k = _blocked(seed, _STREAM["k"], (rows, H, Dk), _l2norm)
    v = _blocked(seed, _STREAM["v"], (rows, H, Dv), np.zeros_like if v_zero else ident)
    g = _blocked(seed, _STREAM["g"], (rows, H, Dk), gmap[g_mode])
    beta = _blocked(seed, _STREAM["beta"], (rows, H), bmap[beta_mode])
    s0 = None
    if init_state:
        s0 = torch.from_numpy(_blocked(seed, _STREAM["s0"], (N, H, Dk, Dv),
                                       lambda x: np.float32(s0_std) * x))
    shp = lambda x: x.reshape((B, T) + x.shape[1:])  # noqa: E731
    return dict(q=_round(shp(q), dtype), k=_round(shp(k), dtype), v=_round(shp(v), dtype),
                g=_round(shp(g), dtype), beta=_round(shp(beta), dtype), initial_state=s0,
                cu_seqlens=None if cu is None else torch.from_numpy(cu))


def make_prologue_inputs(B, T, H, Dk, Dv, seed, dtype="bf16", init_state=False, lengths=None,
                         n_seqs=0, len_lo=0, len_hi=0, param_std=0.5, s0_std=0.02):
    """Raw projections for the fused-prologue forward: the same draws as
    ``make_chunk_inputs`` (same seeds and streams) before any map, i.e. q_raw,
    k_raw, g_logit [B,T,H,Dk] and v [B,T,H,Dv], beta_logit [B,T,H] all N(0,1),
    rounded to ``dtype``; plus the gate parameters A_log [Dk] and dt_bias
    [H*Dk], float32 N(0, param_std^2) from streams 7 and 8. Returns a dict of
    CPU tensors with keys q_raw, k_raw, v, g_logit, beta_logit, A_log, dt_bias,
    initial_state, cu_seqlens."""
    cu = None
    if lengths is None and n_seqs > 0:
        lengths = packed_lengths(np.random.default_rng([seed, _STREAM["lengths"]]), n_seqs, len_lo, len_hi)
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        B, T = 1, int(cu[-1])
    N = B if cu is None else len(cu) - 1
    rows = B * T
    ident = lambda x: x  # noqa: E731
    q = _blocked(seed, _STREAM["q"], (rows, H, Dk), ident)
    k = _blocked(seed, _STREAM["k"], (rows, H, Dk), ident)
    v = _blocked(seed, _STREAM["v"], (rows, H, Dv), ident)
    g = _blocked(seed, _STREAM["g"], (rows, H, Dk), ident)
    beta = _blocked(seed, _STREAM["beta"], (rows, H), ident)
    A_log = (np.float32(param_std) * np.random.default_rng([seed, _STREAM["A_log"]]).standard_normal(
        Dk, dtype=np.float32))
    dt_bias = (np.float32(param_std) * np.random.default_rng([seed, _STREAM["dt_bias"]]).standard_normal(
        H * Dk, dtype=np.float32))
    s0 = None
    if init_state:
        s0 = torch.from_numpy(_blocked(seed, _STREAM["s0"], (N, H, Dk, Dv),
                                       lambda x: np.float32(s0_std) * x))
    shp = lambda x: x.reshape((B, T) + x.shape[1:])  # noqa: E731
    return dict(q_raw=_round(shp(q), dtype), k_raw=_round(shp(k), dtype), v=_round(shp(v), dtype),
                g_logit=_round(shp(g), dtype), beta_logit=_round(shp(beta), dtype),
                A_log=torch.from_numpy(A_log), dt_bias=torch.from_numpy(dt_bias), initial_state=s0,
                cu_seqlens=None if cu is None else torch.from_numpy(cu))


def make_workload(w: Workload, **overrides):
    """Inputs for one of WORKLOADS (overrides go to make_chunk_inputs)."""
    kw = dict(dtype=w.dtype, init_state=w.init_state, n_seqs=w.n_seqs, len_lo=w.len_lo,
              len_hi=w.len_hi)
    kw.update(overrides)
    return make_chunk_inputs(w.B, w.T, w.H, w.Dk, w.Dv, w.seed, **kw)


def make_decode_cache(n_slots, H, Dk, Dv, seed, std=0.02):
    """Decode state cache [n_slots,H,Dk,Dv] float32 ~ N(0, std): stream 6 of
    ``seed``, blocked over slots like every other tensor here."""
    return torch.from_numpy(_blocked(seed, _STREAM["s0"], (n_slots, H, Dk, Dv),
                                     lambda x: np.float32(std) * x))


def make_decode_step(Nb, H, Dk, Dv, seed, step, dtype="bf16"):
    """Token inputs of one decode step, drawn from default_rng([seed, step]).

    q,k [Nb,H,Dk] L2-normalised; v [Nb,H,Dv]; g [Nb,H,Dk] = -5*sigmoid; beta [Nb,H].
    """
    rng = np.random.default_rng([seed, step])
    q = _l2norm(rng.standard_normal((Nb, H, Dk), dtype=np.float32))
    k = _l2norm(rng.standard_normal((Nb, H, Dk), dtype=np.float32))
    v = rng.standard_normal((Nb, H, Dv), dtype=np.float32)
    g = np.float32(GATE_LOWER_BOUND) * _sigmoid(rng.standard_normal((Nb, H, Dk), dtype=np.float32))
    beta = _sigmoid(rng.standard_normal((Nb, H), dtype=np.float32))
    return dict(q=_round(q, dtype), k=_round(k, dtype), v=_round(v, dtype), g=_round(g, dtype),
                beta=_round(beta, dtype))


def make_decode_raw_step(Nb, H, Dk, Dv, seed, step, dtype="bf16"):
    """Raw projections of one decode step, drawn from
    default_rng([seed, 13, step]): q_raw, k_raw, g_logit [Nb,H,Dk], v
    [Nb,H,Dv] and beta_logit [Nb,H], all N(0,1), rounded to ``dtype``. They
    are the inputs of the prologue, or of the short convolution before it."""
    rng = np.random.default_rng([seed, _STREAM["decode_raw"], step])
    f = lambda *shape: rng.standard_normal(shape, dtype=np.float32)  # noqa: E731
    q, k, g = f(Nb, H, Dk), f(Nb, H, Dk), f(Nb, H, Dk)
    v, beta = f(Nb, H, Dv), f(Nb, H)
    return dict(q_raw=_round(q, dtype), k_raw=_round(k, dtype), v=_round(v, dtype), g_logit=_round(g, dtype),
                beta_logit=_round(beta, dtype))


def make_gate_params(H, Dk, seed, std=0.5):
    """The gate's parameters A_log [Dk] and dt_bias [H*Dk], float32
    N(0, std^2), from streams 7 and 8 of ``seed`` (the draws of
    make_prologue_inputs)."""
    A_log = np.float32(std) * np.random.default_rng([seed, _STREAM["A_log"]]).standard_normal(Dk, dtype=np.float32)
    dt_bias = np.float32(std) * np.random.default_rng([seed, _STREAM["dt_bias"]]).standard_normal(
        H * Dk, dtype=np.float32)
    return torch.from_numpy(A_log), torch.from_numpy(dt_bias)


def make_conv_taps(C, seed, which, std=0.5):
    """Short-convolution taps [C,4] float32 N(0, std^2) of projection
    ``which`` (0 q, 1 k, 2 v): default_rng([seed, 11, which])."""
    rng = np.random.default_rng([seed, _STREAM["conv_w"], which])
    return torch.from_numpy(np.float32(std) * rng.standard_normal((C, 4), dtype=np.float32))


def make_conv_cache(n_slots, C, seed, which):
    """Short-convolution cache [n_slots,3,C] float32 N(0,1) of projection
    ``which``: default_rng([seed, 12, which])."""
    rng = np.random.default_rng([seed, _STREAM["conv_cache"], which])
    return torch.from_numpy(rng.standard_normal((n_slots, 3, C), dtype=np.float32))


def as_f32_numpy(t):
    """Exact float32 copy of a CPU tensor (bf16 values are exact in float32)."""
    return None if t is None else t.float().numpy()


def make_cotangents(inp, seed, d_final=True, d_final_std=0.1):
    """Cotangents for the backward of the forward workload ``inp`` (a dict from
    ``make_chunk_inputs``): d_o shaped and typed like the output [B,T,H,Dv] and
    N(0,1), and d_final [N,H,Dk,Dv] float32 N(0, d_final_std^2) or None."""
    B, T, H, Dv = inp["v"].shape
    Dk = inp["q"].shape[-1]
    dtype = "bf16" if inp["v"].dtype == torch.bfloat16 else "f32"
    N = B if inp["cu_seqlens"] is None else inp["cu_seqlens"].numel() - 1
    d_o = _blocked(seed, _STREAM["d_o"], (B * T, H, Dv), lambda x: x).reshape(B, T, H, Dv)
    dfin = None
    if d_final:
        dfin = torch.from_numpy(_blocked(seed, _STREAM["d_final"], (N, H, Dk, Dv),
                                         lambda x: np.float32(d_final_std) * x))
    return _round(d_o, dtype), dfin
