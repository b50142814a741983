"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (default chunk size, bf16, d_k = d_v = 128, H = 96).

Every unit is compared: the GPU runs every head and token, and the fp64 C
oracle (OpenMP over the independent (sequence, head) units on the host's
cores) recomputes all of them. Each (sequence, head) unit must meet the bf16
bar, relL2 <= 2e-2, on its output and on its final state, and so must the
first rows after every sequence start (where the initial state weighs most);
the worst unit is printed. A layout mistake confined to a few heads or
sequences (the silent-garbage failure the hysenlabs article warns of for the
per-channel gate) therefore cannot hide behind a whole-tensor norm.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_chunk_amd as kda
import synth
from oracle import kda_ref
from tests.gpu_helpers import TOL_BF16, rel, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

HEAD_ROWS = 4   # rows after each sequence start checked on their own


def _f(t):
    return None if t is None else t.float().numpy()


def _run_gpu(inp):
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    o, fin = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["initial_state"],
                           cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    kda.device_check()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(fin).all())
    o_h = o.float().cpu().numpy()
    f_h = fin.cpu().numpy()
    del o, fin, d
    torch.cuda.empty_cache()
    return o_h, f_h


def _oracle(inp):
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].numpy().astype(np.int64)
    return kda_ref.c_forward(*(_f(inp[x]) for x in ("q", "k", "v", "g", "beta")),
                             initial_state=_f(inp["initial_state"]), cu_seqlens=cu)


def _per_unit(o, ro, fin, rfin, bounds):
    """relL2 of every (sequence, head) unit: output rows, final state, first rows."""
    H = o.shape[2]
    worst = {"o": (0.0, None), "final": (0.0, None), "first": (0.0, None)}
    for n, (a, b) in enumerate(bounds):
        for h in range(H):
            errs = {"final": rel(fin[n, h], rfin[n, h])}
            if b > a:
                errs["o"] = rel(o[0, a:b, h], ro[0, a:b, h])
                errs["first"] = rel(o[0, a:min(b, a + HEAD_ROWS), h], ro[0, a:min(b, a + HEAD_ROWS), h])
            for key, e in errs.items():
                assert np.isfinite(e) and e <= TOL_BF16, (key, n, h, e)
                if e > worst[key][0]:
                    worst[key] = (e, (n, h))
    return worst


def _report(label, o, ro, fin, rfin, worst, units):
    say(f"        {label}: {units} units; whole-tensor relL2 o={rel(o, ro):.3e} final={rel(fin, rfin):.3e}")
    for key, (e, where) in worst.items():
        say(f"        worst unit {key}: relL2={e:.3e} at (sequence, head)={where}")


@pytest.mark.parametrize("name", ["k3_t4096", "k3_t32768_s0"])
def test_full_size_single_sequence(name):
    w = synth.WORKLOADS[name]
    say(f"[case] full size {name}: B={w.B} T={w.T} H={w.H} d={w.Dk} S0={w.init_state}, every head")
    inp = synth.make_workload(w)
    o, fin = _run_gpu(inp)
    ro, rfin = _oracle(inp)
    worst = _per_unit(o, ro, fin, rfin, [(0, w.T)])
    _report(name, o, ro, fin, rfin, worst, w.H)
    assert rel(o, ro) <= TOL_BF16 and rel(fin, rfin) <= TOL_BF16


def test_full_size_packed_varlen():
    w = synth.WORKLOADS["k3_varlen16"]
    inp = synth.make_workload(w)
    cu = inp["cu_seqlens"].tolist()
    say(f"[case] full size packed: N={len(cu) - 1} T={cu[-1]} H={w.H} lengths={np.diff(cu).tolist()}, "
        f"every (sequence, head)")
    o, fin = _run_gpu(inp)
    ro, rfin = _oracle(inp)
    bounds = list(zip(cu[:-1], cu[1:]))
    worst = _per_unit(o, ro, fin, rfin, bounds)
    _report("k3_varlen16", o, ro, fin, rfin, worst, len(bounds) * w.H)


def test_full_size_decode_128_steps():
    cfg = synth.DECODE
    Nb, H, Dk, Dv, steps, seed = cfg["Nb"], cfg["H"], cfg["Dk"], cfg["Dv"], cfg["steps"], cfg["seed"]
    say(f"[case] full size decode: Nb={Nb} H={H} d={Dk} steps={steps}, every row and head")
    cache = synth.make_decode_cache(Nb, H, Dk, Dv, seed=seed)
    ref = cache.double().numpy()
    dcache = cache.cuda()
    del cache
    outs = np.zeros((steps, Nb, H, Dv), dtype=np.float32)
    refs = np.zeros((steps, Nb, H, Dv))
    for step in range(steps):
        x = synth.make_decode_step(Nb, H, Dk, Dv, seed, step)
        d = {k: v.cuda() for k, v in x.items()}
        o = kda.recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], dcache)
        outs[step] = o.float().cpu().numpy()
        refs[step] = kda_ref.c_decode_step(*(x[n].float().numpy() for n in ("q", "k", "v", "g", "beta")), ref)
    torch.cuda.synchronize()
    kda.device_check()
    got = dcache.cpu().numpy()
    worst_o, worst_c = (0.0, None), (0.0, None)
    for r in range(Nb):
        for h in range(H):
            eo = rel(outs[:, r, h], refs[:, r, h])
            ec = rel(got[r, h], ref[r, h])
            assert eo <= TOL_BF16 and ec <= TOL_BF16, (r, h, eo, ec)
            worst_o = max(worst_o, (eo, (r, h)), key=lambda t: t[0])
            worst_c = max(worst_c, (ec, (r, h)), key=lambda t: t[0])
    say(f"        decode: whole relL2 o(all steps)={rel(outs, refs):.3e} cache={rel(got, ref):.3e}")
    say(f"        worst (row, head) o over the steps: relL2={worst_o[0]:.3e} at {worst_o[1]}; "
        f"cache: relL2={worst_c[0]:.3e} at {worst_c[1]}")


def test_full_size_decode_from_conv_inputs():
    """kda_recurrent_step_conv on the decode workload's shape (256 rows x 96
    heads, d = 128, bf16), 16 steps, every row and head against the oracle's
    chain: the convolution step (float64 caches), the prologue (float64), and
    the C oracle's decode step (which takes the prologue's outputs as float32,
    a 1e-7 relative rounding far below the bar)."""
    cfg = synth.DECODE
    Nb, H, Dk, Dv, seed, steps = cfg["Nb"], cfg["H"], cfg["Dk"], cfg["Dv"], cfg["seed"], 16
    lb, eps = synth.GATE_LOWER_BOUND, 1e-6
    say(f"[case] full size decode from conv inputs: Nb={Nb} H={H} d={Dk} steps={steps}, every row and head")
    cache = synth.make_decode_cache(Nb, H, Dk, Dv, seed=seed)
    ref = cache.double().numpy()
    dcache = cache.cuda()
    del cache
    A_log, dt_bias = synth.make_gate_params(H, Dk, seed)
    Cs = (H * Dk, H * Dk, H * Dv)
    taps = [synth.make_conv_taps(C, seed, j) for j, C in enumerate(Cs)]
    conv0 = [synth.make_conv_cache(Nb, C, seed, j) for j, C in enumerate(Cs)]
    dconv = [c.cuda() for c in conv0]
    rconv = [c.double().numpy().copy() for c in conv0]
    dtaps = [t.cuda() for t in taps]
    dA, db = A_log.cuda(), dt_bias.cuda()
    outs = np.zeros((steps, Nb, H, Dv), dtype=np.float32)
    refs = np.zeros((steps, Nb, H, Dv))
    for step in range(steps):
        x = synth.make_decode_raw_step(Nb, H, Dk, Dv, seed, step)
        d = {k: v.cuda() for k, v in x.items()}
        o = kda.recurrent_step_conv(d["q_raw"], d["k_raw"], d["v"], *dtaps, dconv, d["g_logit"], d["beta_logit"],
                                    dA, db, dcache, gate_lower_bound=lb, l2_eps=eps)
        outs[step] = o.float().cpu().numpy()
        y = [kda_ref.c_short_conv_step(x[n].float().numpy().reshape(Nb, Cs[j]), taps[j].numpy(), rconv[j],
                                       activation=True).reshape(x[n].shape)
             for j, n in enumerate(("q_raw", "k_raw", "v"))]
        q, k, g, beta = kda_ref.prologue(y[0], y[1], x["g_logit"].float().numpy(), x["beta_logit"].float().numpy(),
                                         A_log.numpy(), dt_bias.numpy(), lb, eps)
        refs[step] = kda_ref.c_decode_step(q, k, y[2], g, beta, ref)
    torch.cuda.synchronize()
    kda.device_check()
    got = dcache.cpu().numpy()
    for j in range(3):
        np.testing.assert_array_equal(dconv[j].cpu().numpy().astype(np.float64), rconv[j])
    worst_o, worst_c = (0.0, None), (0.0, None)
    for r in range(Nb):
        for h in range(H):
            eo = rel(outs[:, r, h], refs[:, r, h])
            ec = rel(got[r, h], ref[r, h])
            assert eo <= TOL_BF16 and ec <= TOL_BF16, (r, h, eo, ec)
            worst_o = max(worst_o, (eo, (r, h)), key=lambda t: t[0])
            worst_c = max(worst_c, (ec, (r, h)), key=lambda t: t[0])
    say(f"        decode from conv inputs: whole relL2 o={rel(outs, refs):.3e} cache={rel(got, ref):.3e}")
    say(f"        worst (row, head) o: relL2={worst_o[0]:.3e} at {worst_o[1]}; cache: {worst_c[0]:.3e} at {worst_c[1]}")
