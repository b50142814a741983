"""GPU parity of the backward from raw projections (kda_chunk_bwd_prologue
through the C ABI) against the oracle: its prologue, the C oracle's gradient
of the recurrence, then its prologue gradient, all in float64 on the same
inputs. Every output is float32 from float32 arithmetic, so every tensor is
held to relative L2 <= 1e-4, including dA_log (summed over all tokens and
heads) and ddt_bias (over all tokens).
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_chunk_amd as kda
import synth
from oracle import kda_ref
from tests.gpu_helpers import TOL_F32, rel, say, to_dev

pytestmark = pytest.mark.gpu
NAMES = ("dq_raw", "dk_raw", "dv", "dg_logit", "dbeta_logit", "dA_log", "ddt_bias", "d_initial")
LB, EPS = -5.0, 1e-6


def _cotangents(inp, seed):
    return synth.make_cotangents({"v": inp["v"], "q": inp["q_raw"], "cu_seqlens": inp["cu_seqlens"]}, seed)


def gpu_grads(inp, d_o, d_fin, scale, lb=LB):
    d = to_dev(inp)
    out = kda.chunk_bwd_prologue(d["q_raw"], d["k_raw"], d["v"], d["g_logit"], d["beta_logit"], d["A_log"],
                                 d["dt_bias"], d_o.cuda(), gate_lower_bound=lb, l2_eps=EPS,
                                 initial_state=d["initial_state"],
                                 d_final_state=None if d_fin is None else d_fin.cuda(),
                                 cu_seqlens=d["cu_seqlens"], scale=scale)
    torch.cuda.synchronize()
    return [None if x is None else x.cpu().numpy() for x in out]


def oracle_grads(inp, d_o, d_fin, scale, lb=LB):
    f = lambda t: None if t is None else t.float().numpy().astype(np.float64)  # noqa: E731
    raw = {k: f(inp[k]) for k in ("q_raw", "k_raw", "v", "g_logit", "beta_logit", "A_log", "dt_bias")}
    q, k, g, beta = kda_ref.prologue(raw["q_raw"], raw["k_raw"], raw["g_logit"], raw["beta_logit"], raw["A_log"],
                                     raw["dt_bias"], lb, EPS)
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].numpy().astype(np.int64)
    dq, dk, dv, dg, db, d0 = kda_ref.c_backward(q, k, raw["v"], g, beta, f(d_o), initial_state=f(inp["initial_state"]),
                                                d_final=f(d_fin), cu_seqlens=cu, scale=scale)
    dqr, dkr, dgl, dbl, dA, dbias = kda_ref.prologue_backward(raw["q_raw"], raw["k_raw"], raw["g_logit"],
                                                              raw["beta_logit"], raw["A_log"], raw["dt_bias"],
                                                              dq, dk, dg, db, lb, EPS)
    return [dqr, dkr, dv, dgl, dbl, dA, dbias, d0]


def _check(inp, d_o, d_fin, scale=1.0, label="", lb=LB):
    say(f"[case] bwd prologue {label} q_raw={tuple(inp['q_raw'].shape)} {inp['q_raw'].dtype}")
    got = gpu_grads(inp, d_o, d_fin, scale, lb)
    ref = oracle_grads(inp, d_o, d_fin, scale, lb)
    errs = {n: rel(x, r) for n, x, r in zip(NAMES, got, ref)}
    say("        relL2 " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n, x in zip(NAMES, got):
        assert np.isfinite(x).all(), n
    for n, e in errs.items():
        assert e <= TOL_F32, (n, e)


@pytest.mark.parametrize("B,T,H", [(1, 300, 3), (2, 45, 2)])
def test_bwd_prologue_bf16_k3_dims(B, T, H):
    inp = synth.make_prologue_inputs(B, T, H, 128, 128, seed=700 + T, dtype="bf16", init_state=True)
    d_o, d_fin = _cotangents(inp, 701 + T)
    _check(inp, d_o, d_fin, scale=128 ** -0.5, label=f"bf16 B={B} T={T} H={H}")


@pytest.mark.parametrize("Dk,Dv", [(64, 32), (16, 64), (128, 16)])
def test_bwd_prologue_f32_dims(Dk, Dv):
    inp = synth.make_prologue_inputs(2, 70, 3, Dk, Dv, seed=710 + Dk + Dv, dtype="f32", init_state=True)
    d_o, d_fin = _cotangents(inp, 711)
    _check(inp, d_o, d_fin, scale=0.6, label=f"f32 Dk={Dk} Dv={Dv}")


def test_bwd_prologue_packed_ragged():
    inp = synth.make_prologue_inputs(1, 0, 3, 128, 128, seed=720, dtype="bf16", init_state=True,
                                     lengths=[0, 1, 17, 64, 130, 5])
    d_o, d_fin = _cotangents(inp, 721)
    _check(inp, d_o, d_fin, label="packed")


def test_bwd_prologue_empty_sequences():
    inp = synth.make_prologue_inputs(2, 0, 3, 64, 64, seed=730, dtype="f32", init_state=True)
    d_o, d_fin = _cotangents(inp, 731)
    got = gpu_grads(inp, d_o, d_fin, 1.0)
    np.testing.assert_array_equal(got[5], 0.0)
    np.testing.assert_array_equal(got[6], 0.0)
    np.testing.assert_array_equal(got[7], d_fin.numpy())


def test_bwd_prologue_is_deterministic():
    inp = synth.make_prologue_inputs(1, 400, 4, 128, 128, seed=740, dtype="bf16", init_state=True)
    d_o, d_fin = _cotangents(inp, 741)
    a = gpu_grads(inp, d_o, d_fin, 1.0)
    b = gpu_grads(inp, d_o, d_fin, 1.0)
    for n, x, y in zip(NAMES, a, b):
        assert np.array_equal(x, y), n


@pytest.mark.slow
def test_bwd_prologue_full_k3_shape():
    # B=1, T=4096, H=96, d=128, bf16 raw projections; the oracle runs the whole workload
    # (dA_log sums over every head).
    w = synth.WORKLOADS["k3_t4096"]
    inp = synth.make_prologue_inputs(w.B, w.T, w.H, w.Dk, w.Dv, seed=w.seed, dtype=w.dtype)
    d_o, d_fin = _cotangents(inp, 750)
    _check(inp, d_o, d_fin, scale=128 ** -0.5, label="full k3_t4096")


def test_bwd_prologue_gate_bound_below_five():
    # lb = -8 puts g below -5, outside the matrix-core backward's range: the call
    # takes the vector-ALU backward and still meets the bar.
    inp = synth.make_prologue_inputs(1, 120, 2, 128, 128, seed=760, dtype="bf16", init_state=True)
    d_o, d_fin = _cotangents(inp, 761)
    _check(inp, d_o, d_fin, label="lb=-8", lb=-8.0)


def test_bwd_prologue_bf16_inputs_match_their_float32_widening_bitwise():
    # bf16 raw inputs run the matrix-core backward with float32 q, k, g, beta and bf16 v, dO;
    # the same values widened to float32 run it with every input float32. The arithmetic is
    # the same, so the gradients must agree bit for bit.
    inp = synth.make_prologue_inputs(1, 300, 3, 128, 128, seed=770, dtype="bf16", init_state=True)
    d_o, d_fin = _cotangents(inp, 771)
    wide = {k: (None if v is None or v.dtype != torch.bfloat16 else v.float()) for k, v in inp.items()}
    wide = {k: (wide[k] if wide[k] is not None else inp[k]) for k in inp}
    say("[case] bwd prologue bf16 vs widened float32, T=300 H=3")
    a = gpu_grads(inp, d_o, d_fin, 0.5)
    b = gpu_grads(wide, d_o.float(), d_fin, 0.5)
    for n, x, y in zip(NAMES, a, b):
        assert np.array_equal(x, y), n
