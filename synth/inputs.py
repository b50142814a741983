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

Recipe (all draws from numpy's PCG64 ``default_rng(seed)``, float32):
  draw order: [sequence lengths] -> q -> k -> v -> g_raw -> beta_raw -> [S0]
  q, k  ~ N(0,1), then L2-normalised over d_k per (token, head), in float32
  v     ~ N(0,1)
  g     = -5 * sigmoid(g_raw), g_raw ~ N(0,1)   (per channel, in [-5, 0))
  beta  = sigmoid(beta_raw), beta_raw ~ N(0,1)  (per token and head)
  S0    ~ N(0, 0.02) float32 when requested (0.02 is the standard deviation)
then, for bf16 workloads, q,k,v,g,beta are rounded to bf16 (round to nearest
even). States stay float32.
"""
from __future__ import annotations

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
    rng = np.random.default_rng(seed)
    cu = None
    if lengths is None and n_seqs > 0:
        lengths = packed_lengths(rng, n_seqs, len_lo, len_hi)
    if lengths is not None:
        lengths = np.asarray(lengths, dtype=np.int64)
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        B, T = 1, int(cu[-1])
    N = B if cu is None else len(cu) - 1
    q = _l2norm(rng.standard_normal((B, T, H, Dk), dtype=np.float32))
    k = _l2norm(rng.standard_normal((B, T, H, Dk), dtype=np.float32))
    v = rng.standard_normal((B, T, H, Dv), dtype=np.float32)
    g_raw = rng.standard_normal((B, T, H, Dk), dtype=np.float32)
    b_raw = rng.standard_normal((B, T, H), dtype=np.float32)
    if g_mode == "default":
        g = np.float32(GATE_LOWER_BOUND) * _sigmoid(g_raw)
    elif g_mode == "weak":
        g = np.float32(-0.05) * _sigmoid(g_raw)
    elif g_mode == "zero":
        g = np.zeros_like(g_raw)
    elif g_mode == "bound":
        g = np.full_like(g_raw, GATE_LOWER_BOUND)
    else:
        raise ValueError(g_mode)
    if beta_mode == "default":
        beta = _sigmoid(b_raw)
    elif beta_mode == "one":
        beta = np.ones_like(b_raw)
    elif beta_mode == "zero":
        beta = np.zeros_like(b_raw)
    else:
        raise ValueError(beta_mode)
    if v_zero:
        v = np.zeros_like(v)
    s0 = None
    if init_state:
        s0 = torch.from_numpy(
            (np.float32(s0_std) * rng.standard_normal((N, H, Dk, Dv), dtype=np.float32)))
    return dict(q=_round(q, dtype), k=_round(k, dtype), v=_round(v, dtype), g=_round(g, dtype),
                beta=_round(beta, dtype), initial_state=s0,
                cu_seqlens=None if cu is None else torch.from_numpy(cu))


def make_workload(w: Workload, **overrides):
    """Inputs for one of WORKLOADS (overrides go to make_chunk_inputs)."""
    kw = dict(dtype=w.dtype, init_state=w.init_state, n_seqs=w.n_seqs, len_lo=w.len_lo,
              len_hi=w.len_hi)
    kw.update(overrides)
    return make_chunk_inputs(w.B, w.T, w.H, w.Dk, w.Dv, w.seed, **kw)


def make_decode_cache(n_slots, H, Dk, Dv, seed, std=0.02):
    """Decode state cache [n_slots,H,Dk,Dv] float32 ~ N(0, std), from default_rng(seed)."""
    rng = np.random.default_rng(seed)
    return torch.from_numpy(np.float32(std) * rng.standard_normal((n_slots, H, Dk, Dv),
                                                                  dtype=np.float32))


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


def as_f32_numpy(t):
    """Exact float32 copy of a CPU tensor (bf16 values are exact in float32)."""
    return None if t is None else t.float().numpy()
