"""GPU parity of the backward from the pre-convolution projections
(kda_chunk_bwd_conv): bit for bit against the sequence of calls it stands
for (the three convolutions, kda_chunk_bwd_prologue, kda_short_conv_bwd per
projection), and against the fp64 oracle's chain (convolution -> prologue ->
recurrence and their gradients) at the backward's bar, relative L2 <= 1e-4.
Cotangents of the final conv states are included.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_chunk_amd as kda
import synth
from oracle import kda_ref
from tests.gpu_helpers import TOL_F32, rel, say

pytestmark = pytest.mark.gpu

LB, EPS = -5.0, 1e-6
NAMES = ("q_raw", "k_raw", "v")


def _case(B, T, H, Dk, Dv, seed, dtype, lengths=None):
    inp = synth.make_prologue_inputs(B, T, H, Dk, Dv, seed=seed, dtype=dtype, init_state=True, lengths=lengths)
    B, T = inp["q_raw"].shape[:2]
    N = B if inp["cu_seqlens"] is None else inp["cu_seqlens"].numel() - 1
    Cs = (H * Dk, H * Dk, H * Dv)
    taps = [synth.make_conv_taps(C, seed, j) for j, C in enumerate(Cs)]
    rng = np.random.default_rng([seed, 99])
    s0 = [torch.from_numpy(rng.standard_normal((N, 3, C)).astype(np.float32)) for C in Cs]
    dfin = [torch.from_numpy((0.1 * rng.standard_normal((N, 3, C))).astype(np.float32)) for C in Cs]
    cot = {"v": inp["v"], "q": inp["q_raw"], "cu_seqlens": inp["cu_seqlens"]}
    d_o, d_fin = synth.make_cotangents(cot, seed + 1)
    return inp, taps, s0, dfin, d_o, d_fin, Cs


def _gpu_fused(inp, taps, s0, dfin, d_o, d_fin, scale):
    dev = "cuda"
    d = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    return kda.chunk_bwd_conv(d["q_raw"], d["k_raw"], d["v"], *(t.to(dev) for t in taps), d["g_logit"],
                              d["beta_logit"], d["A_log"], d["dt_bias"], d_o.to(dev),
                              conv_states=[t.to(dev) for t in s0], d_conv_final=[t.to(dev) for t in dfin],
                              gate_lower_bound=LB, l2_eps=EPS, initial_state=d["initial_state"],
                              d_final_state=d_fin.to(dev), cu_seqlens=d["cu_seqlens"], scale=scale)


@pytest.mark.parametrize("dtype,packed,Dk,Dv", [("bf16", False, 128, 128), ("f32", False, 128, 128),
                                                ("bf16", True, 128, 128), ("f32", True, 128, 128),
                                                ("f32", False, 64, 32), ("bf16", True, 32, 64)])
def test_bwd_conv_equals_the_sequence_of_calls_bitwise(dtype, packed, Dk, Dv):
    H, scale = 2, Dk ** -0.5
    lengths = [37, 0, 64, 100] if packed else None
    inp, taps, s0, dfin, d_o, d_fin, Cs = _case(2, 77, H, Dk, Dv, seed=1400, dtype=dtype, lengths=lengths)
    B, T = inp["q_raw"].shape[:2]
    say(f"[case] bwd conv == chain, {dtype} B={B} T={T} packed={packed}")
    got = _gpu_fused(inp, taps, s0, dfin, d_o, d_fin, scale)

    dev = "cuda"
    d = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    cu = d["cu_seqlens"]
    ys = {}
    for j, n in enumerate(NAMES):
        ys[n], _ = kda.short_conv(d[n], taps[j].to(dev), conv_state=s0[j].to(dev), cu_seqlens=cu, activation=True,
                                  output_final_state=False)
        ys[n] = ys[n].reshape(d[n].shape)
    dqr, dkr, dv, dgl, dbl, dA, dbias, d0 = kda.chunk_bwd_prologue(
        ys["q_raw"], ys["k_raw"], ys["v"], d["g_logit"], d["beta_logit"], d["A_log"], d["dt_bias"], d_o.to(dev),
        gate_lower_bound=LB, l2_eps=EPS, initial_state=d["initial_state"], d_final_state=d_fin.to(dev),
        cu_seqlens=cu, scale=scale)
    ref = {"g_logit": dgl, "beta_logit": dbl, "A_log": dA, "dt_bias": dbias, "initial_state": d0}
    for j, (n, dy, key) in enumerate(zip(NAMES, (dqr, dkr, dv), "qkv")):
        dx, dw, dst = kda.short_conv_bwd(d[n], taps[j].to(dev), dy.reshape(B, T, Cs[j]).contiguous(),
                                         conv_state=s0[j].to(dev), d_final_state=dfin[j].to(dev), cu_seqlens=cu,
                                         activation=True)
        ref.update({"x" + key: dx.reshape(got["x" + key].shape), "w" + key: dw, "conv_state_" + key: dst})
    torch.cuda.synchronize()
    for k, v in ref.items():
        assert torch.equal(got[k], v), k


def test_bwd_conv_against_oracle_chain():
    B, T, H, D, scale = 2, 90, 2, 128, 128 ** -0.5
    inp, taps, s0, dfin, d_o, d_fin, Cs = _case(B, T, H, D, D, seed=1410, dtype="f32")
    say(f"[case] bwd conv against the oracle chain, f32 B={B} T={T}")
    got = _gpu_fused(inp, taps, s0, dfin, d_o, d_fin, scale)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in got.items()}

    f = lambda t: t.float().numpy().astype(np.float64)  # noqa: E731
    ry = {n: kda_ref.short_conv(f(inp[n]).reshape(B, T, Cs[j]), f(taps[j]), f(s0[j]), activation=True)[0]
          .reshape(B, T, H, D) for j, n in enumerate(NAMES)}
    raw = {k: f(inp[k]) for k in ("g_logit", "beta_logit", "A_log", "dt_bias")}
    q, k, g, beta = kda_ref.prologue(ry["q_raw"], ry["k_raw"], raw["g_logit"], raw["beta_logit"], raw["A_log"],
                                     raw["dt_bias"], LB, EPS)
    dq, dk, rdv, dg, db, rd0 = kda_ref.c_backward(q, k, ry["v"], g, beta, f(d_o), initial_state=f(inp["initial_state"]),
                                                  d_final=f(d_fin), scale=scale)
    rdqr, rdkr, rdgl, rdbl, rdA, rdbias = kda_ref.prologue_backward(ry["q_raw"], ry["k_raw"], raw["g_logit"],
                                                                    raw["beta_logit"], raw["A_log"], raw["dt_bias"],
                                                                    dq, dk, dg, db, LB, EPS)
    ref = {"g_logit": rdgl, "beta_logit": rdbl, "A_log": rdA, "dt_bias": rdbias, "initial_state": rd0}
    for j, (n, dy, key) in enumerate(zip(NAMES, (rdqr, rdkr, rdv), "qkv")):
        dx, dw, dst = kda_ref.short_conv_backward(f(inp[n]).reshape(B, T, Cs[j]), f(taps[j]), dy.reshape(B, T, Cs[j]),
                                                  f(s0[j]), d_final=f(dfin[j]), activation=True)
        ref.update({"x" + key: dx, "w" + key: dw, "conv_state_" + key: dst})
    errs = {k: rel(got[k].reshape(ref[k].shape), ref[k]) for k in ref}
    say("        relL2 " + " ".join(f"{k}={e:.2e}" for k, e in errs.items()))
    for k, e in errs.items():
        assert np.isfinite(got[k]).all(), k
        assert e <= TOL_F32, (k, e)
