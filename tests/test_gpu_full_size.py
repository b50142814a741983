"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (default chunk size, bf16, d_k = d_v = 128, H = 96).

The GPU runs every head and token. The fp64 oracle recomputes a sample of the
independent (sequence, head) units in full, and the comparison covers every
output and final-state element of those units. Bars: relL2 <= 2e-2 for bf16
inputs, per tensor, plus the same bar on the rows right after each sequence
start (where the initial state weighs most).
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_chunk_amd as kda
import synth
from oracle import kda_ref
from tests.gpu_helpers import TOL_BF16, rel, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

HEADS = [0, 41, 95]


def _f(t):
    return None if t is None else t.float().numpy()


def _heads(t, hs):
    return None if t is None else t[:, :, hs].contiguous()


def _run_gpu(inp):
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    o, fin = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["initial_state"],
                           cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(fin).all())
    return o, fin


def _oracle_units(inp, hs, a, b, n):
    """Oracle over tokens [a, b) of sequence n for heads hs."""
    sl = {x: inp[x][:, a:b] for x in ("q", "k", "v", "g", "beta")}
    s0 = inp["initial_state"]
    s0 = None if s0 is None else s0[n:n + 1, hs].contiguous().numpy()
    return kda_ref.c_forward(*(_f(_heads(sl[x], hs)) for x in ("q", "k", "v", "g")),
                             _f(sl["beta"][:, :, hs].contiguous()), initial_state=s0)


def _compare(o_gpu, f_gpu, ro, rf, label, head_rows=4):
    eo, ef = rel(o_gpu, ro), rel(f_gpu, rf)
    es = rel(o_gpu[:, :head_rows], ro[:, :head_rows])
    say(f"        {label}: relL2 o={eo:.3e} final={ef:.3e} first{head_rows}={es:.3e}")
    assert eo <= TOL_BF16 and ef <= TOL_BF16 and es <= TOL_BF16, (eo, ef, es)


@pytest.mark.parametrize("name", ["k3_t4096", "k3_t32768_s0"])
def test_full_size_single_sequence(name):
    w = synth.WORKLOADS[name]
    say(f"[case] full size {name}: B={w.B} T={w.T} H={w.H} d={w.Dk} S0={w.init_state}")
    inp = synth.make_workload(w)
    o, fin = _run_gpu(inp)
    o_s = o[:, :, HEADS].float().cpu().numpy()
    f_s = fin[:, HEADS].cpu().numpy()
    del o, fin
    ro, rf = _oracle_units(inp, HEADS, 0, w.T, 0)
    _compare(o_s, f_s, ro, rf, f"heads {HEADS}")


def test_full_size_packed_varlen():
    w = synth.WORKLOADS["k3_varlen16"]
    inp = synth.make_workload(w)
    cu = inp["cu_seqlens"].tolist()
    say(f"[case] full size packed: N={len(cu) - 1} T={cu[-1]} H={w.H} lengths={np.diff(cu).tolist()}")
    o, fin = _run_gpu(inp)
    lens = np.diff(cu)
    picks = sorted({int(np.argmax(lens)), int(np.argmin(lens)), 0, len(lens) - 1})
    for n, hs in zip(picks, ([0, 95], [17], [63], [40, 41])):
        a, b = cu[n], cu[n + 1]
        o_s = o[:, a:b][:, :, hs].float().cpu().numpy()
        f_s = fin[n:n + 1, hs].cpu().numpy()
        ro, rf = _oracle_units(inp, hs, a, b, n)
        _compare(o_s, f_s, ro, rf, f"sequence {n} (len {b - a}) heads {hs}")


def test_full_size_decode_128_steps():
    cfg = synth.DECODE
    Nb, H, Dk, Dv, steps, seed = cfg["Nb"], cfg["H"], cfg["Dk"], cfg["Dv"], cfg["steps"], cfg["seed"]
    rows = [0, 77, 200, 255]
    say(f"[case] full size decode: Nb={Nb} H={H} d={Dk} steps={steps}, oracle rows {rows}")
    cache = synth.make_decode_cache(Nb, H, Dk, Dv, seed=seed)
    ref = cache[rows].double().numpy().copy()
    dcache = cache.cuda()
    del cache
    outs, refs = [], []
    for step in range(steps):
        x = synth.make_decode_step(Nb, H, Dk, Dv, seed, step)
        d = {k: v.cuda() for k, v in x.items()}
        o = kda.recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], dcache)
        outs.append(o[rows].float().cpu().numpy())
        refs.append(kda_ref.c_decode_step(*(x[n][rows].float().numpy() for n in ("q", "k", "v", "g", "beta")),
                                          ref))
    torch.cuda.synchronize()
    eo = rel(np.stack(outs), np.stack(refs))
    ec = rel(dcache[rows].cpu().numpy(), ref)
    say(f"        decode relL2 o(all steps)={eo:.3e} cache={ec:.3e}")
    assert eo <= TOL_BF16 and ec <= TOL_BF16
