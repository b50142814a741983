"""Shared helpers for the GPU parity tests (GPU path vs the fp64 oracle)."""
import sys

import numpy as np
import torch

import gated_delta_rule_chunk_amd as kda
from oracle import kda_ref

# Parity bars (relative L2 over whole tensors): fp32 inputs, bf16 inputs
TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(inp, device="cuda"):
    out = {}
    for key, val in inp.items():
        out[key] = None if val is None else val.to(device)
    return out


def gpu_chunk(inp, chunk=0, scale=1.0, final=True):
    d = to_dev(inp)
    o, fin = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["initial_state"],
                           cu_seqlens=d["cu_seqlens"], chunk_size=chunk, scale=scale,
                           output_final_state=final)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), (None if fin is None else fin.cpu().numpy())


def oracle_chunk(inp, scale=1.0, heads=None, nthreads=0):
    """C oracle on the exact inputs; ``heads`` restricts it to a subset of heads."""
    f = lambda t: None if t is None else t.float().numpy()  # noqa: E731
    q, k, v, g, beta = (f(inp[x]) for x in ("q", "k", "v", "g", "beta"))
    s0 = f(inp["initial_state"])
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].numpy().astype(np.int64)
    if heads is not None:
        q, k, v, g = (x[:, :, heads] for x in (q, k, v, g))
        beta = beta[:, :, heads]
        if s0 is not None:
            s0 = s0[:, heads]
    return kda_ref.c_forward(q, k, v, g, beta, initial_state=s0, cu_seqlens=cu, scale=scale,
                             nthreads=nthreads)


def rel(x, ref):
    return kda_ref.rel_l2(x, ref)
