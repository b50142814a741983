"""Pins for the oracle's gradient of the short causal convolution.

Central differences of ``short_conv`` itself (pinned in
test_oracle_conv_pins.py) check every entry of dx, dw and the conv-state
gradient, with and without SiLU, on packed batches that include sequences
shorter than the kernel (whose final state reaches into the initial state).
Closed forms fix the transposed taps (an impulse in dy comes back through the
taps in reverse order) and the weight gradient of a linear convolution.
Planted mistakes fail.
"""
import numpy as np
import pytest

from oracle import kda_ref


def _case(seed, B, T, C, N=None):
    rng = np.random.default_rng(seed)
    N = B if N is None else N
    f = lambda *s: np.asarray(rng.standard_normal(s), dtype=np.float32).astype(np.float64)  # noqa: E731
    return f(B, T, C), f(C, 4), f(N, 3, C), f(B, T, C), f(N, 3, C)


def _loss(x, w, st, dy, dfin, cu, act):
    y, fin = kda_ref.short_conv(x, w, st, cu_seqlens=cu, activation=act)
    return float((y * dy).sum() + (fin * dfin).sum())


@pytest.mark.parametrize("act", [False, True])
@pytest.mark.parametrize("packed", [False, True])
def test_every_gradient_matches_central_differences(act, packed):
    if packed:
        x, w, st, dy, dfin = _case(1, 1, 11, 3, N=4)
        cu = np.array([0, 2, 2, 7, 11])          # lengths 2, 0, 5, 4
    else:
        x, w, st, dy, dfin = _case(2, 2, 6, 3)
        cu = None
    dx, dw, dst = kda_ref.short_conv_backward(x, w, dy, st, dfin, cu_seqlens=cu, activation=act)
    eps = 1e-6
    for name, base, got in (("x", x, dx), ("w", w, dw), ("state", st, dst)):
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            args = {"x": x, "w": w, "state": st}
            plus, minus = dict(args), dict(args)
            plus[name], minus[name] = base.copy(), base.copy()
            plus[name][idx] += eps
            minus[name][idx] -= eps
            fd[idx] = (_loss(plus["x"], plus["w"], plus["state"], dy, dfin, cu, act)
                       - _loss(minus["x"], minus["w"], minus["state"], dy, dfin, cu, act)) / (2 * eps)
        np.testing.assert_allclose(got, fd, rtol=0, atol=2e-8 * max(1.0, np.abs(fd).max()), err_msg=name)


def test_impulse_comes_back_through_reversed_taps():
    C, T = 4, 12
    w = np.random.default_rng(3).standard_normal((C, 4))
    x = np.zeros((1, T, C))
    dy = np.zeros((1, T, C))
    dy[0, 6] = 1.0
    dx, dw, dst = kda_ref.short_conv_backward(x, w, dy)
    for t in range(T):
        expect = w[:, t - 3] if 3 <= t <= 6 else np.zeros(C)    # y[6] = sum_i w[:, i] x[3 + i]
        np.testing.assert_allclose(dx[0, t], expect, rtol=0, atol=1e-15)
    np.testing.assert_array_equal(dst, 0.0)


def test_linear_weight_gradient_is_a_cross_correlation():
    x, w, _, dy, _ = _case(4, 1, 9, 2)
    _, dw, _ = kda_ref.short_conv_backward(x, w, dy)
    ext = np.concatenate([np.zeros((3, 2)), x[0]], axis=0)
    expect = np.stack([(dy[0] * ext[i:i + 9]).sum(0) for i in range(4)], axis=1)
    np.testing.assert_allclose(dw, expect, rtol=1e-13)


@pytest.mark.parametrize("mistake", ["taps_forward", "no_silu_slope", "final_to_first"])
def test_planted_mistakes_fail(mistake):
    x, w, st, dy, dfin = _case(5, 1, 8, 2)
    act = mistake == "no_silu_slope"
    dx, dw, dst = kda_ref.short_conv_backward(x, w, dy, st, dfin, activation=act)
    if mistake == "taps_forward":                 # taps applied in forward instead of reversed order
        bad = kda_ref.short_conv_backward(x, w[:, ::-1].copy(), dy, st, dfin, activation=act)[0]
    elif mistake == "no_silu_slope":              # SiLU's derivative taken as sigmoid alone
        y_lin, _ = kda_ref.short_conv(x, w, st)
        sg = 1.0 / (1.0 + np.exp(-y_lin))
        bad = kda_ref.short_conv_backward(x, w, dy * sg, st, dfin)[0]
    else:                                         # final-state cotangent sent to the first tokens
        bad = kda_ref.short_conv_backward(x, w, dy, st, None)[0]
        bad[0, :3] += dfin[0]
    eps = 1e-6
    idx = (0, 5, 1)
    xp, xm = x.copy(), x.copy()
    xp[idx] += eps
    xm[idx] -= eps
    fd = (_loss(xp, w, st, dy, dfin, None, act) - _loss(xm, w, st, dy, dfin, None, act)) / (2 * eps)
    assert abs(dx[idx] - fd) < 1e-7
    assert abs(bad[idx] - fd) > 1e-5
