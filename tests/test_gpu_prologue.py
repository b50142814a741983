"""GPU parity of the fused gate, beta and normalisation prologue
(kda_chunk_fwd_prologue) against the fp64 oracle's prologue forward.

Inputs are raw projections (q, k unnormalised, gate and beta logits) with the
gate parameters A_log [Dk] and dt_bias [H*Dk]; both kernels (the float32 chunk
kernel and the bf16 matrix-core kernel) are covered, over several chunks with
ragged tails, packed sequences, initial states and saturated gates. The bar is
the forward's: relative L2 over whole tensors, fp32 <= 1e-4, bf16 <= 2e-2.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_chunk_amd as kda
import synth
from oracle import kda_ref
from tests.gpu_helpers import TOL_BF16, TOL_F32, rel, say, to_dev

pytestmark = pytest.mark.gpu

LB, EPS = -5.0, 1e-6


def gpu_prologue(inp, chunk=0, scale=1.0, lb=LB, eps=EPS):
    d = to_dev(inp)
    o, fin = kda.chunk_fwd_prologue(d["q_raw"], d["k_raw"], d["v"], d["g_logit"], d["beta_logit"], d["A_log"],
                                    d["dt_bias"], gate_lower_bound=lb, l2_eps=eps,
                                    initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"],
                                    chunk_size=chunk, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), fin.cpu().numpy()


def oracle_prologue(inp, scale=1.0, lb=LB, eps=EPS, heads=None):
    f = lambda t: None if t is None else t.float().numpy()  # noqa: E731
    q, k, v, g, b = (f(inp[x]) for x in ("q_raw", "k_raw", "v", "g_logit", "beta_logit"))
    A_log, dt_bias, s0 = f(inp["A_log"]), f(inp["dt_bias"]), f(inp["initial_state"])
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].numpy().astype(np.int64)
    if heads is not None:
        H, Dk = q.shape[2], q.shape[3]
        q, k, v, g = (x[:, :, heads] for x in (q, k, v, g))
        b = b[:, :, heads]
        dt_bias = dt_bias.reshape(H, Dk)[heads].reshape(-1)
        if s0 is not None:
            s0 = s0[:, heads]
    return kda_ref.c_prologue_forward(q, k, v, g, b, A_log, dt_bias, lb, eps, initial_state=s0,
                                      cu_seqlens=cu, scale=scale)


def _check(inp, tol, chunk=0, scale=1.0, lb=LB, eps=EPS, label=""):
    say(f"[case] prologue {label} chunk={chunk} q={tuple(inp['q_raw'].shape)} {inp['q_raw'].dtype} lb={lb}")
    o, fin = gpu_prologue(inp, chunk=chunk, scale=scale, lb=lb, eps=eps)
    ro, rfin = oracle_prologue(inp, scale=scale, lb=lb, eps=eps)
    eo, ef = rel(o, ro), rel(fin, rfin)
    say(f"        relL2 o={eo:.3e} final={ef:.3e}")
    assert np.isfinite(o).all() and np.isfinite(fin).all()
    assert eo <= tol and ef <= tol, (eo, ef)


@pytest.mark.parametrize("Dk,Dv,chunk", [(32, 64, 16), (128, 128, 64), (64, 16, 32), (16, 128, 64)])
def test_f32_general_dims(Dk, Dv, chunk):
    inp = synth.make_prologue_inputs(2, 150, 3, Dk, Dv, seed=500 + Dk + Dv, dtype="f32", init_state=True,
                                     s0_std=0.5)
    _check(inp, TOL_F32, chunk=chunk, label=f"f32 Dk={Dk} Dv={Dv}")


def test_bf16_general_path():
    inp = synth.make_prologue_inputs(1, 170, 4, 64, 64, seed=601, dtype="bf16", init_state=True)
    _check(inp, TOL_BF16, chunk=32, label="bf16 generic 64x64")


@pytest.mark.parametrize("B,T,H", [(1, 293, 5), (3, 200, 16), (1, 1, 3), (3, 77, 96)])
def test_bf16_d128(B, T, H):
    inp = synth.make_prologue_inputs(B, T, H, 128, 128, seed=700 + T + H, dtype="bf16", init_state=True)
    _check(inp, TOL_BF16, label=f"bf16 d128 B={B} T={T} H={H}")


@pytest.mark.parametrize("H", [8, 3])
def test_bf16_packed_ragged(H):
    inp = synth.make_prologue_inputs(1, 0, H, 128, 128, seed=800 + H, dtype="bf16", init_state=True,
                                     lengths=[0, 1, 63, 64, 65, 130, 7, 257])
    _check(inp, TOL_BF16, label=f"bf16 packed H={H}")


def test_f32_packed_ragged():
    inp = synth.make_prologue_inputs(1, 0, 4, 64, 32, seed=811, dtype="f32", init_state=True,
                                     lengths=[5, 0, 64, 100, 1])
    _check(inp, TOL_F32, chunk=16, label="f32 packed")


@pytest.mark.parametrize("mode", ["saturated_gate", "large_eps", "scaled_output"])
def test_bf16_d128_stress(mode):
    inp = synth.make_prologue_inputs(1, 211, 6, 128, 128, seed=900 + len(mode), dtype="bf16", init_state=True)
    kw = {}
    if mode == "saturated_gate":
        # logits far from the bias: gates at the bound (every decay e^-5) or at 0
        inp["g_logit"] = (inp["g_logit"].float() * 40.0).to(torch.bfloat16)
    elif mode == "large_eps":
        kw["eps"] = 30.0          # comparable to |q|^2 ~ 128: the eps term matters
    else:
        kw["scale"] = 128 ** -0.5
    _check(inp, TOL_BF16, label=f"bf16 d128 {mode}", **kw)


@pytest.mark.parametrize("lb", [-8.0, -1.0])
def test_other_gate_bounds(lb):
    # below -5 the bf16 d=128 call runs the float32 kernel (the matrix-core one
    # needs g >= -5); above it, either kernel
    inp = synth.make_prologue_inputs(1, 150, 4, 128, 128, seed=950, dtype="bf16", init_state=True)
    _check(inp, TOL_BF16, lb=lb, label=f"bf16 d128 lb={lb}")


def test_full_size_k3_t4096_every_head():
    w = synth.WORKLOADS["k3_t4096"]
    inp = synth.make_prologue_inputs(w.B, w.T, w.H, w.Dk, w.Dv, seed=w.seed, dtype="bf16")
    say(f"[case] prologue full size k3_t4096, every head")
    o, fin = gpu_prologue(inp)
    ro, rf = oracle_prologue(inp)
    assert np.isfinite(o).all() and np.isfinite(fin).all()
    worst = (0.0, None)
    for h in range(w.H):
        eo, ef = rel(o[:, :, h], ro[:, :, h]), rel(fin[:, h], rf[:, h])
        assert eo <= TOL_BF16 and ef <= TOL_BF16, (h, eo, ef)
        worst = max(worst, (max(eo, ef), h), key=lambda t: t[0])
    say(f"        whole relL2 o={rel(o, ro):.3e} final={rel(fin, rf):.3e}; worst head {worst[1]} at {worst[0]:.3e}")


# --- the prologue on its own (kda_prologue) ------------------------------------

@pytest.mark.parametrize("dtype,Dk", [("bf16", 128), ("f32", 128), ("f32", 32), ("bf16", 16)])
def test_standalone_prologue_against_oracle(dtype, Dk):
    inp = synth.make_prologue_inputs(2, 70, 3, Dk, Dk, seed=560 + Dk, dtype=dtype)
    say(f"[case] kda_prologue {dtype} Dk={Dk}")
    d = to_dev(inp)
    q, k, g, b = kda.prologue(d["q_raw"], d["k_raw"], d["g_logit"], d["beta_logit"], d["A_log"], d["dt_bias"],
                              gate_lower_bound=LB, l2_eps=EPS)
    torch.cuda.synchronize()
    f = lambda t: t.float().numpy()  # noqa: E731
    ref = kda_ref.prologue(f(inp["q_raw"]), f(inp["k_raw"]), f(inp["g_logit"]), f(inp["beta_logit"]),
                           f(inp["A_log"]), f(inp["dt_bias"]), LB, EPS)
    # float32: rounding only; bf16: one rounding of each output to bf16 (2^-8 relative at most)
    tol = 4e-3 if dtype == "bf16" else 1e-6
    for name, got, r in zip("qkgb", (q, k, g, b), ref):
        e = rel(got.float().cpu().numpy(), r)
        say(f"        {name}: relL2 {e:.2e}")
        assert e <= tol, (name, e)
    # in place: each output over its own input gives the same values
    q2, k2, g2, b2 = (t.clone() for t in (d["q_raw"], d["k_raw"], d["g_logit"], d["beta_logit"]))
    kda.prologue(q2, k2, g2, b2, d["A_log"], d["dt_bias"], gate_lower_bound=LB, l2_eps=EPS, out=(q2, k2, g2, b2))
    torch.cuda.synchronize()
    for a_, b_ in ((q2, q), (k2, k), (g2, g), (b2, b)):
        assert torch.equal(a_, b_)


def test_standalone_prologue_then_chunk_forward_matches_the_fused_call():
    """float32: kda_prologue then kda_chunk_fwd against kda_chunk_fwd_prologue
    (the same function; the gate's rounding differs between the two kernels)."""
    inp = synth.make_prologue_inputs(1, 150, 2, 64, 64, seed=570, dtype="f32", init_state=True)
    d = to_dev(inp)
    q, k, g, b = kda.prologue(d["q_raw"], d["k_raw"], d["g_logit"], d["beta_logit"], d["A_log"], d["dt_bias"],
                              gate_lower_bound=LB, l2_eps=EPS)
    o1, f1 = kda.chunk_fwd(q, k, d["v"], g, b, initial_state=d["initial_state"])
    o2, f2 = gpu_prologue(inp)
    eo, ef = rel(o1.cpu().numpy(), o2), rel(f1.cpu().numpy(), f2)
    say(f"[case] kda_prologue -> kda_chunk_fwd vs fused: relL2 o={eo:.2e} final={ef:.2e}")
    assert eo <= 1e-5 and ef <= 1e-5
