"""Pins for the oracle's gradient through the gate, beta and L2-norm prologue.

The composed map raw projections -> prologue -> recurrence is differentiated by
chaining ``recurrence_backward`` (pinned in test_oracle_backward_pins.py) with
``prologue_backward``; central differences of the composed forward check every
input, including the gate parameters A_log and dt_bias, which are shared across
tokens (and, for A_log, across heads). Closed forms fix the normalisation's
scale invariance and the gate's and beta's slopes at zero. Planted mistakes
fail the pins.
"""
import numpy as np
import pytest

from oracle import kda_ref

NAMES = ("q_raw", "k_raw", "g_logit", "beta_logit", "A_log", "dt_bias")
LB, EPS = -5.0, 1e-6


def _case(seed, B=1, T=7, H=2, Dk=4, Dv=3):
    rng = np.random.default_rng(seed)
    f = lambda *shape: np.asarray(rng.standard_normal(shape), dtype=np.float32).astype(np.float64)  # noqa: E731
    raw = dict(q_raw=f(B, T, H, Dk), k_raw=f(B, T, H, Dk), g_logit=f(B, T, H, Dk), beta_logit=f(B, T, H),
               A_log=0.5 * f(Dk), dt_bias=0.5 * f(H * Dk))
    return raw, f(B, T, H, Dv), f(B, T, H, Dv), f(B, H, Dk, Dv), f(B, H, Dk, Dv)


def _loss(raw, v, s0, d_o, d_fin, scale):
    q, k, g, beta = kda_ref.prologue(raw["q_raw"], raw["k_raw"], raw["g_logit"], raw["beta_logit"], raw["A_log"],
                                     raw["dt_bias"], LB, EPS)
    o, fin = kda_ref.recurrence(q, k, v, g, beta, s0, scale=scale)
    return float((o * d_o).sum() + (fin * d_fin).sum())


def _grads(raw, v, s0, d_o, d_fin, scale, backward=None):
    q, k, g, beta = kda_ref.prologue(raw["q_raw"], raw["k_raw"], raw["g_logit"], raw["beta_logit"], raw["A_log"],
                                     raw["dt_bias"], LB, EPS)
    dq, dk, dv, dg, db, d0 = kda_ref.recurrence_backward(q, k, v, g, beta, d_o, s0, d_fin, scale=scale)
    back = backward or kda_ref.prologue_backward
    return back(raw["q_raw"], raw["k_raw"], raw["g_logit"], raw["beta_logit"], raw["A_log"], raw["dt_bias"],
                dq, dk, dg, db, LB, EPS)


def test_every_raw_gradient_matches_central_differences():
    raw, v, d_o, s0, d_fin = _case(1)
    scale = 0.8
    got = _grads(raw, v, s0, d_o, d_fin, scale)
    eps = 1e-6
    for name, value in zip(NAMES, got):
        base = raw[name]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            plus, minus = dict(raw), dict(raw)
            plus[name], minus[name] = base.copy(), base.copy()
            plus[name][idx] += eps
            minus[name][idx] -= eps
            fd[idx] = (_loss(plus, v, s0, d_o, d_fin, scale) - _loss(minus, v, s0, d_o, d_fin, scale)) / (2 * eps)
        np.testing.assert_allclose(value, fd, rtol=0, atol=3e-8 * max(1.0, np.abs(fd).max()), err_msg=name)


def test_normalisation_gradient_is_almost_orthogonal_to_the_row():
    # q = x / sqrt(|x|^2 + eps) is scale invariant up to eps: x . dx = (x . dq) eps / n^3 exactly.
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 3, 8))
    dq = rng.standard_normal((5, 3, 8))
    eps = 0.3
    zeros = np.zeros((5, 3, 8))
    dx = kda_ref.prologue_backward(x, x, zeros, np.zeros((5, 3)), np.zeros(8), np.zeros(24), dq, dq, zeros,
                                   np.zeros((5, 3)), LB, eps)[0]
    n = np.sqrt((x * x).sum(-1) + eps)
    np.testing.assert_allclose((x * dx).sum(-1), (x * dq).sum(-1) * eps / n ** 3, rtol=1e-12)


def test_gate_and_beta_slopes_at_zero():
    # At z = 0 the gate's slope is lb/4 per unit of logit (A_log = 0: rate 1), and beta's is 1/4;
    # dt_bias collects the same slope, A_log gets dz * z = 0.
    H, Dk = 2, 3
    zeros = np.zeros((1, 1, H, Dk))
    ones = np.ones((1, 1, H, Dk))
    out = kda_ref.prologue_backward(zeros + 1.0, zeros + 1.0, zeros, np.zeros((1, 1, H)), np.zeros(Dk),
                                    np.zeros(H * Dk), zeros, zeros, ones, np.ones((1, 1, H)), LB, EPS)
    np.testing.assert_allclose(out[2], LB / 4)
    np.testing.assert_allclose(out[3], 0.25)
    np.testing.assert_allclose(out[5], LB / 4)
    np.testing.assert_allclose(out[4], 0.0, atol=0)


@pytest.mark.parametrize("mistake", ["no_cube", "no_A", "bias_per_channel_only"])
def test_planted_mistakes_fail(mistake):
    raw, v, d_o, s0, d_fin = _case(3, T=5, H=2, Dk=3, Dv=2)

    def wrong(q_raw, k_raw, g_logit, beta_logit, A_log, dt_bias, dq, dk, dg, dbeta, lb, eps):
        out = list(kda_ref.prologue_backward(q_raw, k_raw, g_logit, beta_logit, A_log, dt_bias, dq, dk, dg, dbeta,
                                             lb, eps))
        n = np.sqrt((q_raw * q_raw).sum(-1, keepdims=True) + eps)
        if mistake == "no_cube":       # dropping the projection term of the norm's derivative
            out[0] = dq / n
        elif mistake == "no_A":        # forgetting the rate exp(A_log) in the logit's gradient
            out[2] = out[2] / np.exp(A_log)
        else:                          # dt_bias summed over heads as if shared like A_log
            H = q_raw.shape[-2]
            out[5] = np.tile(out[5].reshape(H, -1).sum(0), H)
        return tuple(out)

    good = _grads(raw, v, s0, d_o, d_fin, 0.7)
    bad = _grads(raw, v, s0, d_o, d_fin, 0.7, backward=wrong)
    assert any(not np.allclose(a, b, rtol=1e-6, atol=1e-9) for a, b in zip(good, bad))
    # and the central difference decides for the right one
    eps = 1e-6
    name = {"no_cube": "q_raw", "no_A": "g_logit", "bias_per_channel_only": "dt_bias"}[mistake]
    i = NAMES.index(name)
    base = raw[name]
    idx = tuple(0 for _ in base.shape)
    plus, minus = dict(raw), dict(raw)
    plus[name], minus[name] = base.copy(), base.copy()
    plus[name][idx] += eps
    minus[name][idx] -= eps
    fd = (_loss(plus, v, s0, d_o, d_fin, 0.7) - _loss(minus, v, s0, d_o, d_fin, 0.7)) / (2 * eps)
    assert abs(good[i][idx] - fd) < 1e-7 * max(1.0, abs(fd))
    assert abs(bad[i][idx] - fd) > 1e-6 * max(1.0, abs(fd))
