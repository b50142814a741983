"""Pins for the oracle's reverse-mode gradient of the KDA recurrence.

The gradient is the derivative of the forward recurrence (already pinned on
its own) for the loss L = sum_t <d_o[t], o[t]> + <d_final, S_T>. The pins here
do not reuse the backward formulas: central finite differences of the forward
oracle check every gradient output entry by entry; closed forms fix the
single-token case and the pure-decay case (beta = 0); the C and NumPy forms,
written separately, must agree, including across the C form's 64-token
checkpoint blocks and with ragged, empty and packed sequences. A planted sign
or index mistake in the gradient fails the finite-difference test.
"""
import numpy as np
import pytest

from oracle import kda_ref


def _c_built():
    try:
        kda_ref.load_c()
        return True
    except RuntimeError:
        return False


needs_c = pytest.mark.skipif(not _c_built(), reason="C oracle not built")
GRADS = [kda_ref.recurrence_backward] + ([kda_ref.c_backward] if _c_built() else [])
NAMES = ("q", "k", "v", "g", "beta", "initial_state")


def _f32(a):
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _case(seed, B, T, H, Dk, Dv, N=None):
    rng = np.random.default_rng(seed)
    N = B if N is None else N
    q = _f32(rng.standard_normal((B, T, H, Dk)))
    k = _f32(rng.standard_normal((B, T, H, Dk)) / np.sqrt(Dk))
    v = _f32(rng.standard_normal((B, T, H, Dv)))
    g = _f32(-rng.uniform(0.0, 0.8, (B, T, H, Dk)))
    beta = _f32(rng.uniform(0.1, 0.95, (B, T, H)))
    s0 = _f32(rng.standard_normal((N, H, Dk, Dv)))
    d_o = _f32(rng.standard_normal((B, T, H, Dv)))
    d_fin = _f32(rng.standard_normal((N, H, Dk, Dv)))
    return dict(q=q, k=k, v=v, g=g, beta=beta, initial_state=s0), d_o, d_fin


def _loss(args, d_o, d_fin, cu, scale):
    o, fin = kda_ref.recurrence(args["q"], args["k"], args["v"], args["g"], args["beta"],
                                args["initial_state"], cu_seqlens=cu, scale=scale)
    return float((o * d_o).sum() + (fin * d_fin).sum())


def _finite_difference(args, d_o, d_fin, cu, scale, name, eps=1e-6):
    base = args[name]
    fd = np.zeros_like(base)
    for idx in np.ndindex(base.shape):
        plus = dict(args)
        minus = dict(args)
        plus[name] = base.copy()
        minus[name] = base.copy()
        plus[name][idx] += eps
        minus[name][idx] -= eps
        fd[idx] = (_loss(plus, d_o, d_fin, cu, scale) - _loss(minus, d_o, d_fin, cu, scale)) / (2 * eps)
    return fd


@pytest.mark.parametrize("grad", GRADS)
@pytest.mark.parametrize("varlen", [False, True])
def test_every_gradient_matches_central_differences(grad, varlen):
    if varlen:
        args, d_o, d_fin = _case(3, 1, 9, 2, 4, 3, N=3)
        cu = np.array([0, 4, 4, 9])                        # includes an empty sequence
    else:
        args, d_o, d_fin = _case(2, 2, 6, 2, 4, 3)
        cu = None
    scale = 0.6
    got = grad(args["q"], args["k"], args["v"], args["g"], args["beta"], d_o,
               args["initial_state"], d_fin, cu_seqlens=cu, scale=scale)
    for name, value in zip(NAMES, got):
        fd = _finite_difference(args, d_o, d_fin, cu, scale, name)
        np.testing.assert_allclose(value, fd, rtol=0, atol=2e-8 * max(1.0, np.abs(fd).max()),
                                   err_msg=f"d{name}")


def test_single_token_from_zero_state_closed_form():
    # S_1 = beta k v^T, o = scale beta (q.k) v, L = <d_o, o>:
    # dq = scale beta (v.d_o) k, dk = scale beta (v.d_o) q, dv = scale beta (q.k) d_o,
    # dbeta = scale (q.k)(v.d_o), and dg = 0 because the decayed state is zero.
    args, d_o, _ = _case(5, 1, 1, 3, 6, 4)
    q, k, v, g, beta = (args[n][0, 0] for n in NAMES[:5])
    do = d_o[0, 0]
    scale = 0.3
    for grad in GRADS:
        dq, dk, dv, dg, db, _ = grad(args["q"], args["k"], args["v"], args["g"], args["beta"], d_o,
                                     None, None, scale=scale)
        qk = (q * k).sum(-1)
        vdo = (v * do).sum(-1)
        np.testing.assert_allclose(dq[0, 0], scale * (beta * vdo)[:, None] * k, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(dk[0, 0], scale * (beta * vdo)[:, None] * q, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(dv[0, 0], scale * (beta * qk)[:, None] * do, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(db[0, 0], scale * qk * vdo, rtol=1e-12, atol=1e-14)
        np.testing.assert_array_equal(dg[0, 0], 0.0)


def test_pure_decay_closed_form():
    # beta = 0: S_t = Diag(exp G_t) S_0 with G_t the running sum of g, so
    # L = sum_t scale q_t^T Diag(exp G_t) S_0 d_o_t and dL/dg_s[i] =
    # sum_{t >= s} scale q_t[i] exp(G_t[i]) (S_0 d_o_t)[i]; dv = 0, dk = 0.
    args, d_o, _ = _case(6, 1, 7, 2, 5, 3)
    args["beta"][:] = 0.0
    scale = 0.9
    q, g, s0 = args["q"][0], args["g"][0], args["initial_state"][0]
    G = np.cumsum(g, axis=0)                                       # [T,H,Dk]
    s0do = np.einsum("hkv,thv->thk", s0, d_o[0])                   # S_0 d_o_t
    terms = scale * q * np.exp(G) * s0do                           # [T,H,Dk]
    dg_expect = np.cumsum(terms[::-1], axis=0)[::-1]
    dq_expect = scale * np.exp(G) * s0do
    d0_expect = scale * np.einsum("thk,thv->hkv", np.exp(G) * q, d_o[0])
    for grad in GRADS:
        dq, dk, dv, dg, db, d0 = grad(args["q"], args["k"], args["v"], args["g"], args["beta"], d_o,
                                      args["initial_state"], None, scale=scale)
        np.testing.assert_allclose(dg[0], dg_expect, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(dq[0], dq_expect, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(d0[0], d0_expect, rtol=1e-12, atol=1e-13)
        np.testing.assert_array_equal(dv, 0.0)
        np.testing.assert_allclose(dk, 0.0, atol=0)


def test_final_state_only_loss_is_the_transposed_recurrence():
    # With d_o = 0 the gradient with respect to the initial state is the
    # adjoint map of the state transition: <d_final, S_T> is linear in S_0, so
    # <d_initial, Z> equals <d_final, S_T(S_0 + Z) - S_T(S_0)> for any Z.
    args, d_o, d_fin = _case(7, 1, 12, 2, 4, 3)
    d_o[:] = 0.0
    for grad in GRADS:
        d0 = grad(args["q"], args["k"], args["v"], args["g"], args["beta"], d_o,
                  args["initial_state"], d_fin)[5]
        Z = np.random.default_rng(8).standard_normal(d0.shape)
        _, f1 = kda_ref.recurrence(args["q"], args["k"], args["v"], args["g"], args["beta"],
                                   args["initial_state"] + Z)
        _, f0 = kda_ref.recurrence(args["q"], args["k"], args["v"], args["g"], args["beta"],
                                   args["initial_state"])
        np.testing.assert_allclose((d0 * Z).sum(), (d_fin * (f1 - f0)).sum(), rtol=1e-11)


@needs_c
def test_c_and_numpy_agree_across_checkpoint_blocks_and_ragged_sequences():
    # The C form re-runs each 64-token block from a checkpoint; lengths 0, 1,
    # 63, 64, 65 and 150 cover every block edge.
    lens = [0, 1, 63, 64, 65, 150]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    args, d_o, d_fin = _case(9, 1, T, 2, 8, 6, N=len(lens))
    a = kda_ref.recurrence_backward(args["q"], args["k"], args["v"], args["g"], args["beta"], d_o,
                                    args["initial_state"], d_fin, cu_seqlens=cu, scale=0.4)
    b = kda_ref.c_backward(args["q"], args["k"], args["v"], args["g"], args["beta"], d_o,
                           args["initial_state"], d_fin, cu_seqlens=cu, scale=0.4, nthreads=2)
    for name, x, y in zip(NAMES, a, b):
        np.testing.assert_allclose(y, x, rtol=1e-10, atol=1e-11 * max(1.0, np.abs(x).max()),
                                   err_msg=f"d{name}")


@needs_c
def test_c_long_sequence_sampled_central_differences():
    # One 150-token sequence (three checkpoint blocks): central differences of
    # the loss at a few sampled entries of each input, against the C gradient.
    args, d_o, d_fin = _case(10, 1, 150, 1, 4, 3)
    got = kda_ref.c_backward(args["q"], args["k"], args["v"], args["g"], args["beta"], d_o,
                             args["initial_state"], d_fin, scale=0.5)
    rng = np.random.default_rng(11)
    eps = 1e-6
    for name, value in zip(NAMES, got):
        base = args[name]
        for _ in range(4):
            idx = tuple(int(rng.integers(0, s)) for s in base.shape)
            plus, minus = dict(args), dict(args)
            plus[name] = base.copy()
            minus[name] = base.copy()
            plus[name][idx] += eps
            minus[name][idx] -= eps
            fd = (_loss(plus, d_o, d_fin, None, 0.5) - _loss(minus, d_o, d_fin, None, 0.5)) / (2 * eps)
            assert abs(value[idx] - fd) <= 1e-7 * max(1.0, abs(fd)), (name, idx, value[idx], fd)


@needs_c
def test_c_rejects_bad_arguments():
    args, d_o, _ = _case(12, 1, 5, 1, 3, 2, N=2)
    with pytest.raises(ValueError):
        kda_ref.c_backward(args["q"], args["k"], args["v"], args["g"], args["beta"], d_o,
                           cu_seqlens=np.array([0, 3, 4]))            # does not end at T
    with pytest.raises(ValueError):
        kda_ref.c_backward(args["q"], args["k"], args["v"], args["g"], args["beta"], d_o,
                           cu_seqlens=np.array([0, 4, 3, 5]))         # decreasing
