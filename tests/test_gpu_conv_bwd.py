"""GPU parity of the short convolution's backward (kda_short_conv_bwd through
the C ABI) against the fp64 oracle's gradient on the same inputs, and of the
whole backward from pre-convolution projections (convolution -> prologue ->
recurrence, then back) against the oracle's chain. The gradients are float32
from float32 arithmetic on exactly representable inputs (bf16 inputs are
widened exactly), so every tensor is held to relative L2 <= 1e-4 whatever the
input dtype.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_chunk_amd as kda
import synth
from oracle import kda_ref
from tests.gpu_helpers import TOL_F32, rel, say

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _inputs(B, T, C, dtype, seed, lengths=None, state=True, d_final=True):
    rng = np.random.default_rng(seed)
    cu = None
    if lengths is not None:
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        B, T = 1, int(cu[-1])
    N = B if cu is None else len(lengths)
    f = lambda *s: torch.from_numpy(rng.standard_normal(s).astype(np.float32))  # noqa: E731
    x = f(B, T, C).to(DT[dtype])
    w = 0.5 * f(C, 4)
    s0 = f(N, 3, C) if state else None
    dy = f(B, T, C)
    dfin = f(N, 3, C) if d_final else None
    return dict(x=x, w=w, s0=s0, cu=None if cu is None else torch.from_numpy(cu), dy=dy, dfin=dfin)


def gpu_grads(c, act):
    dev = "cuda"
    d = {k: None if v is None else v.to(dev) for k, v in c.items()}
    dx, dw, dst = kda.short_conv_bwd(d["x"], d["w"], d["dy"], conv_state=d["s0"], d_final_state=d["dfin"],
                                     cu_seqlens=d["cu"], activation=act)
    torch.cuda.synchronize()
    return dx.cpu().numpy(), dw.cpu().numpy(), dst.cpu().numpy()


def oracle_grads(c, act):
    f = lambda t: None if t is None else t.float().numpy().astype(np.float64)  # noqa: E731
    cu = None if c["cu"] is None else c["cu"].numpy().astype(np.int64)
    dx, dw, dst = kda_ref.short_conv_backward(f(c["x"]), f(c["w"]), f(c["dy"]), f(c["s0"]), f(c["dfin"]),
                                              cu_seqlens=cu, activation=act)
    return dx, dw, dst


def _check(c, act, label):
    say(f"[case] conv bwd {label} x={tuple(c['x'].shape)} {c['x'].dtype} act={act} "
        f"state={c['s0'] is not None} d_final={c['dfin'] is not None}")
    got = gpu_grads(c, act)
    ref = oracle_grads(c, act)
    errs = [rel(g, r) for g, r in zip(got, ref)]
    say("        relL2 dx={:.2e} dw={:.2e} d_state={:.2e}".format(*errs))
    for g in got:
        assert np.isfinite(g).all()
    assert max(errs) <= TOL_F32, errs


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("act", [True, False])
@pytest.mark.parametrize("B,T,C", [(2, 150, 256), (1, 33, 12288), (3, 5, 64), (1, 200, 2056)])
def test_conv_bwd(dtype, act, B, T, C):
    c = _inputs(B, T, C, dtype, seed=B * 1000 + T + C)
    _check(c, act, f"B={B} T={T} C={C}")


@pytest.mark.parametrize("state,d_final", [(True, True), (False, True), (True, False), (False, False)])
def test_conv_bwd_packed_ragged(state, d_final):
    # empty, one-, two- and three-token sequences (whose windows reach into the
    # initial state) between longer ones, some crossing 64-token blocks
    c = _inputs(1, 0, 384, "bf16", seed=88, lengths=[0, 1, 2, 3, 17, 0, 40, 16, 130, 2, 64, 1, 0],
                state=state, d_final=d_final)
    _check(c, True, "packed")


def test_conv_bwd_empty_batch():
    c = _inputs(2, 0, 64, "f32", seed=89)
    dx, dw, dst = gpu_grads(c, True)
    assert dx.size == 0
    np.testing.assert_array_equal(dw, 0.0)
    np.testing.assert_array_equal(dst, c["dfin"].numpy())   # the final window is the initial state


def test_conv_bwd_is_deterministic():
    c = _inputs(1, 3000, 512, "bf16", seed=90)
    a = gpu_grads(c, True)
    b = gpu_grads(c, True)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.slow
def test_conv_bwd_full_projection_width():
    # one projection of the B=1, T=4096, H=96, d=128 workload: C = 12288 channels, bf16, SiLU
    c = _inputs(1, 4096, 96 * 128, "bf16", seed=91)
    _check(c, True, "full T=4096 C=12288")


def test_backward_from_pre_convolution_projections():
    """q, k, v through the convolution (SiLU), the fused-prologue forward's
    backward, then the convolution's backward: the GPU chain against the
    oracle's float64 chain (convolution, prologue, recurrence and their
    gradients), every gradient of the pre-convolution inputs and parameters."""
    B, T, H, D = 1, 150, 2, 128
    inp = synth.make_prologue_inputs(B, T, H, D, D, seed=1300, dtype="f32", init_state=True)
    rng = np.random.default_rng(1301)
    C = H * D
    conv_w = {n: torch.from_numpy((0.5 * rng.standard_normal((C, 4))).astype(np.float32))
              for n in ("q_raw", "k_raw", "v")}
    conv_s0 = {n: torch.from_numpy(rng.standard_normal((B, 3, C)).astype(np.float32)) for n in conv_w}
    d_o, d_fin = synth.make_cotangents({"v": inp["v"], "q": inp["q_raw"], "cu_seqlens": None}, 1302)
    lb, eps, scale = -5.0, 1e-6, D ** -0.5
    dev = "cuda"

    # GPU chain
    ys = {}
    for n in conv_w:
        ys[n], _ = kda.short_conv(inp[n].to(dev), conv_w[n].to(dev), conv_state=conv_s0[n].to(dev),
                                  activation=True, output_final_state=False)
        ys[n] = ys[n].reshape(B, T, H, D)
    dqr, dkr, dv, dgl, dbl, dA, dbias, d0 = kda.chunk_bwd_prologue(
        ys["q_raw"], ys["k_raw"], ys["v"], inp["g_logit"].to(dev), inp["beta_logit"].to(dev),
        inp["A_log"].to(dev), inp["dt_bias"].to(dev), d_o.to(dev), gate_lower_bound=lb, l2_eps=eps,
        initial_state=inp["initial_state"].to(dev), d_final_state=d_fin.to(dev), scale=scale)
    got = {"g_logit": dgl, "beta_logit": dbl, "A_log": dA, "dt_bias": dbias, "initial_state": d0}
    for n, dy in (("q_raw", dqr), ("k_raw", dkr), ("v", dv)):
        dx, dw, dst = kda.short_conv_bwd(inp[n].to(dev), conv_w[n].to(dev), dy.reshape(B, T, C).contiguous(),
                                         conv_state=conv_s0[n].to(dev), activation=True)
        got.update({f"x_{n}": dx, f"w_{n}": dw, f"s0_{n}": dst})
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in got.items()}

    # oracle chain, float64
    f = lambda t: t.float().numpy().astype(np.float64)  # noqa: E731
    ry = {n: kda_ref.short_conv(f(inp[n]).reshape(B, T, C), f(conv_w[n]), f(conv_s0[n]), activation=True)[0]
          .reshape(B, T, H, D) for n in conv_w}
    raw = {k: f(inp[k]) for k in ("g_logit", "beta_logit", "A_log", "dt_bias")}
    q, k, g, beta = kda_ref.prologue(ry["q_raw"], ry["k_raw"], raw["g_logit"], raw["beta_logit"], raw["A_log"],
                                     raw["dt_bias"], lb, eps)
    dq, dk, rdv, dg, db, rd0 = kda_ref.c_backward(q, k, ry["v"], g, beta, f(d_o), initial_state=f(inp["initial_state"]),
                                                  d_final=f(d_fin), scale=scale)
    rdqr, rdkr, rdgl, rdbl, rdA, rdbias = kda_ref.prologue_backward(ry["q_raw"], ry["k_raw"], raw["g_logit"],
                                                                    raw["beta_logit"], raw["A_log"], raw["dt_bias"],
                                                                    dq, dk, dg, db, lb, eps)
    ref = {"g_logit": rdgl, "beta_logit": rdbl, "A_log": rdA, "dt_bias": rdbias, "initial_state": rd0}
    for n, dy in (("q_raw", rdqr), ("k_raw", rdkr), ("v", rdv)):
        dx, dw, dst = kda_ref.short_conv_backward(f(inp[n]).reshape(B, T, C), f(conv_w[n]), dy.reshape(B, T, C),
                                                  f(conv_s0[n]), activation=True)
        ref.update({f"x_{n}": dx, f"w_{n}": dw, f"s0_{n}": dst})

    errs = {k: rel(got[k].reshape(ref[k].shape), ref[k]) for k in ref}
    say("[case] conv -> prologue -> recurrence backward: relL2 "
        + " ".join(f"{k}={e:.2e}" for k, e in errs.items()))
    for k, e in errs.items():
        assert np.isfinite(got[k]).all(), k
        assert e <= TOL_F32, (k, e)
