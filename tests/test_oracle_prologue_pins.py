"""Pins for the oracle's gate, beta and normalisation prologue.

The pages fix the gate's parameters and bound but not its formula (hysenlabs
"kimi-k3-mlx", section "The A_log shape mismatch is a silent-garbage bug the
tests assert": A_log per key channel, shared by the heads, dt_bias per (head,
channel); section "Attention is 93 layers ...": gate_lower_bound -5). The
reading pinned here is g = lb * sigmoid(exp(A_log) * (logit + dt_bias)),
beta = sigmoid(beta logit), q and k scaled to x / sqrt(|x|^2 + eps). Each pin
rests on a value the mathematics fixes, not on re-typing the formula: the
closed forms go through the C forward (where only the recurrence's output
reveals the gate), the two implementations are checked against each other,
and a constructed input reduces the prologue path to the already pinned plain
recurrence.
"""
import math

import numpy as np
import pytest

from oracle import kda_ref

LB = -5.0


def _c_built():
    try:
        kda_ref.load_c()
        return True
    except RuntimeError:
        return False


needs_c = pytest.mark.skipif(not _c_built(), reason="C oracle not built")


def _two_token_inputs(H=1, Dk=8, Dv=4, seed=0):
    """Two tokens whose keys are orthogonal basis vectors and whose queries are
    the first key: with a zero initial state,
        o_1 = beta_1 (q^ . k^_1) v_1,  o_2 = exp(g_2[0]) o_1
    since token 2 neither reads nor erases channel 0 (k^_2 = e_1)."""
    rng = np.random.default_rng(seed)
    q = np.zeros((1, 2, H, Dk)); k = np.zeros((1, 2, H, Dk))
    q[:, :, :, 0] = 2.0                      # |q| = 2  -> q^ = 2/sqrt(4+eps) e_0
    k[:, 0, :, 0] = 3.0                      # k^_1 = 3/sqrt(9+eps) e_0
    k[:, 1, :, 1] = 5.0                      # k^_2 = 5/sqrt(25+eps) e_1
    v = rng.standard_normal((1, 2, H, Dv))
    A_log = rng.uniform(-1.0, 1.0, Dk)
    dt_bias = rng.uniform(-2.0, 2.0, H * Dk)
    return q, k, v, A_log, dt_bias


@needs_c
@pytest.mark.parametrize("z, sig", [(0.0, 0.5), (math.log(3.0), 0.75), (-math.log(3.0), 0.25)])
def test_gate_and_beta_closed_forms_through_c_forward(z, sig):
    eps = 1e-6
    q, k, v, A_log, dt_bias = _two_token_inputs()
    H, Dk = q.shape[2], q.shape[3]
    # pre-activation z on channel 0 of token 2: logit = z / exp(A_log[0]) - dt_bias[0]
    glog = np.zeros((1, 2, H, Dk))
    glog[0, 1, :, 0] = z / math.exp(A_log[0]) - dt_bias.reshape(H, Dk)[:, 0]
    blog = np.full((1, 2, H), math.log(3.0))   # beta = sigmoid(ln 3) = 3/4
    o, _ = kda_ref.c_prologue_forward(q, k, v, glog, blog, A_log, dt_bias, LB, eps)
    # f32 holds A_log, dt_bias and the logit: compare against the exact forms on
    # those f32 values
    A0 = float(np.float32(A_log[0]))
    z32 = math.exp(A0) * (float(np.float32(glog[0, 1, 0, 0])) + float(np.float32(dt_bias[0])))
    bl32 = float(np.float32(math.log(3.0)))
    beta = 1.0 / (1.0 + math.exp(-bl32))          # sigmoid of the f32-held ln 3
    assert abs(beta - 0.75) < 1e-7
    cq, ck = 2.0 / math.sqrt(4.0 + eps), 3.0 / math.sqrt(9.0 + eps)
    v32 = v.astype(np.float32).astype(np.float64)
    o1 = beta * cq * ck * v32[0, 0]
    np.testing.assert_allclose(o[0, 0], o1, rtol=1e-12, atol=1e-15)
    g2 = LB / (1.0 + math.exp(-z32))
    assert abs(z32 - z) < 1e-5 and abs(1.0 / (1.0 + math.exp(-z)) - sig) < 1e-15
    np.testing.assert_allclose(o[0, 1], math.exp(g2) * o1, rtol=1e-12, atol=1e-15)


def test_gate_range_and_limits():
    rng = np.random.default_rng(1)
    H, Dk = 3, 16
    A_log = rng.uniform(-1, 1, Dk)
    dt_bias = rng.uniform(-3, 3, H * Dk)
    x = rng.uniform(-2, 2, (5, H, Dk))        # |z| <= e*5: no saturation in float64
    _, _, g, _ = kda_ref.prologue(x, x, x, np.zeros((5, H)), A_log, dt_bias, LB)
    assert np.all(g < 0.0) and np.all(g > LB)
    # monotone: a larger logit decays more (lb < 0)
    _, _, g_up, _ = kda_ref.prologue(x, x, x + 0.5, np.zeros((5, H)), A_log, dt_bias, LB)
    assert np.all(g_up < g)
    # saturation: logits far above / below the bias give lb / 0
    big = np.full((1, H, Dk), 200.0)          # |z| >= 200/e: saturated, no overflow
    _, _, g_hi, _ = kda_ref.prologue(big, big, big, np.zeros((1, H)), A_log, dt_bias, LB)
    _, _, g_lo, _ = kda_ref.prologue(big, big, -big, np.zeros((1, H)), A_log, dt_bias, LB)
    np.testing.assert_allclose(g_hi, LB, rtol=0, atol=1e-12)
    np.testing.assert_allclose(g_lo, 0.0, rtol=0, atol=1e-12)
    # the per-channel A_log is shared by the heads: equal logits+bias on two
    # heads give equal gates, whatever the head
    same = np.zeros((1, H, Dk)) - dt_bias.reshape(1, H, Dk) + 0.3
    _, _, g_same, _ = kda_ref.prologue(same, same, same, np.zeros((1, H)), A_log, dt_bias, LB)
    np.testing.assert_allclose(g_same[0, 0], g_same[0, 1], rtol=1e-15, atol=0)


def test_l2_normalisation_and_beta():
    rng = np.random.default_rng(2)
    H, Dk, eps = 4, 32, 1e-6
    x = rng.standard_normal((7, H, Dk)) * rng.uniform(0.01, 10.0, (7, H, 1))
    q, k, _, beta = kda_ref.prologue(x, 3.0 * x, x, np.array([[0.0, math.log(3.0), -math.log(3.0), 50.0]] * 7),
                                     np.zeros(Dk), np.zeros(H * Dk), LB, eps)
    n2 = (x * x).sum(-1)
    np.testing.assert_allclose((q * q).sum(-1), n2 / (n2 + eps), rtol=1e-12)
    # direction kept: q is a positive multiple of x
    np.testing.assert_allclose(q * np.sqrt(n2 + eps)[..., None], x, rtol=1e-12, atol=1e-15)
    # scaling the input by 3 rescales the output by 3 sqrt(n2 + eps) / sqrt(9 n2 + eps)
    ratio = 3.0 * np.sqrt(n2 + eps) / np.sqrt(9.0 * n2 + eps)
    np.testing.assert_allclose(k, q * ratio[..., None], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(beta[0], [0.5, 0.75, 0.25, 1.0 / (1.0 + math.exp(-50.0))], rtol=1e-15)


@needs_c
def test_c_and_numpy_prologue_paths_agree():
    rng = np.random.default_rng(3)
    B, T, H, Dk, Dv = 2, 37, 3, 16, 8
    q = rng.standard_normal((B, T, H, Dk)).astype(np.float32)
    k = rng.standard_normal((B, T, H, Dk)).astype(np.float32)
    v = rng.standard_normal((B, T, H, Dv)).astype(np.float32)
    gl = rng.standard_normal((B, T, H, Dk)).astype(np.float32)
    bl = rng.standard_normal((B, T, H)).astype(np.float32)
    A_log = rng.uniform(-1, 1, Dk).astype(np.float32)
    dt_bias = rng.uniform(-1, 1, H * Dk).astype(np.float32)
    s0 = (0.1 * rng.standard_normal((B, H, Dk, Dv))).astype(np.float32)
    o_c, f_c = kda_ref.c_prologue_forward(q, k, v, gl, bl, A_log, dt_bias, LB, 1e-6, initial_state=s0)
    qn, kn, g, beta = kda_ref.prologue(q, k, gl, bl, A_log, dt_bias, LB, 1e-6)
    o_n, f_n = kda_ref.recurrence(qn, kn, v, g, beta, initial_state=s0)
    assert kda_ref.rel_l2(o_c, o_n) < 1e-12 and kda_ref.rel_l2(f_c, f_n) < 1e-12


@needs_c
def test_prologue_path_reduces_to_the_plain_recurrence():
    """Raw inputs built to invert the prologue (unit q and k with eps = 0,
    logits solving lb*sigmoid(logit) = g with A_log = dt_bias = 0, beta logits
    = logit(beta)) give the plain oracle's result on (q, k, v, g, beta)."""
    rng = np.random.default_rng(4)
    B, T, H, Dk, Dv = 1, 45, 2, 16, 16
    q = rng.standard_normal((B, T, H, Dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((B, T, H, Dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    g = rng.uniform(-4.9, -0.01, (B, T, H, Dk))
    beta = rng.uniform(0.05, 0.95, (B, T, H))
    glog = -np.log(LB / g - 1.0)
    blog = np.log(beta / (1.0 - beta))
    # feed both paths the same float32 values: the plain path gets the prologue
    # applied (in float64) to the float32 raw inputs
    q32, k32, v32, gl32, bl32 = (a.astype(np.float32) for a in (q, k, v, glog, blog))
    o_p, f_p = kda_ref.c_prologue_forward(q32, k32, v32, gl32, bl32, np.zeros(Dk), np.zeros(H * Dk), LB, 0.0)
    qn, kn, gn, bn = kda_ref.prologue(q32, k32, gl32, bl32, np.zeros(Dk), np.zeros(H * Dk), LB, 0.0)
    # the prologue's outputs are close to the targets ...
    assert np.abs(gn - g).max() < 1e-5 and np.abs(bn - beta).max() < 1e-6
    # ... and through the plain C oracle (which takes float32) agree with the
    # prologue path to float32 rounding of its inputs
    o_r, f_r = kda_ref.c_forward(qn, kn, v32, gn, bn)
    assert kda_ref.rel_l2(o_p, o_r) < 1e-6 and kda_ref.rel_l2(f_p, f_r) < 1e-6


def _pins_hold(prologue_fn):
    """The closed forms and properties above, as one predicate over a prologue
    implementation with kda_ref.prologue's signature."""
    rng = np.random.default_rng(5)
    H, Dk, eps = 2, 8, 1e-6
    A_log = rng.uniform(-1, 1, Dk)
    dt_bias = rng.uniform(-1, 1, H * Dk)
    ok = True
    for z, frac in ((0.0, 0.5), (math.log(3.0), 0.75)):
        logit = (z / np.exp(A_log))[None, None, :] - dt_bias.reshape(1, H, Dk)
        x = rng.standard_normal((1, H, Dk))
        q, _, g, beta = prologue_fn(x, x, logit, np.full((1, H), z), A_log, dt_bias, LB, eps)
        ok &= np.allclose(g, LB * frac, rtol=1e-12, atol=0)
        ok &= np.allclose(beta, frac, rtol=1e-12, atol=0)
        n2 = (x * x).sum(-1)
        ok &= np.allclose((q * q).sum(-1), n2 / (n2 + eps), rtol=1e-12)
    return bool(ok)


def _mistaken(kind):
    def fn(q_raw, k_raw, g_logit, beta_logit, A_log, dt_bias, lb=-5.0, eps=1e-6):
        q_raw, k_raw, g_logit = (np.asarray(a, dtype=np.float64) for a in (q_raw, k_raw, g_logit))
        H, Dk = q_raw.shape[-2:]
        A = np.exp(np.asarray(A_log, dtype=np.float64))
        bias = np.asarray(dt_bias, dtype=np.float64).reshape(H, Dk)
        nq = np.sqrt((q_raw * q_raw).sum(-1, keepdims=True) + eps)
        if kind == "norm_without_sqrt":
            nq = (q_raw * q_raw).sum(-1, keepdims=True) + eps
        q = q_raw / nq
        k = k_raw / np.sqrt((k_raw * k_raw).sum(-1, keepdims=True) + eps)
        z = A * (g_logit + bias)
        if kind == "bias_dropped":
            z = A * g_logit
        if kind == "A_log_per_head":       # A_log broadcast over the head axis instead of the channel axis
            z = A[:H, None] * (g_logit + bias)
        if kind == "softplus_gate":
            z = np.log1p(A) * (g_logit + bias)
        s = 1.0 / (1.0 + np.exp(-z))
        if kind == "sigmoid_sign":
            s = 1.0 / (1.0 + np.exp(z))
        g = (lb if kind != "bound_dropped" else -1.0) * s
        beta = 1.0 / (1.0 + np.exp(-np.asarray(beta_logit, dtype=np.float64)))
        return q, k, g, beta
    return fn


def test_prologue_pins_hold_for_the_oracle():
    assert _pins_hold(kda_ref.prologue)


@pytest.mark.parametrize("kind", ["norm_without_sqrt", "bias_dropped", "A_log_per_head", "softplus_gate",
                                  "sigmoid_sign", "bound_dropped"])
def test_prologue_planted_mistakes_are_caught(kind):
    assert not _pins_hold(_mistaken(kind))
