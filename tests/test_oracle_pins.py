"""Pins for the fp64 oracle, checked against facts other than the oracle itself.

Each pin is chosen so that a plausible mistake in the oracle (a dropped term, a
wrong sign, decay and erase in the wrong order, output read before the update,
a transposed state, a per-head instead of per-channel decay) fails at least one
of them; ``test_planted_mistakes_are_caught`` plants those mistakes in copies
of the oracle's token step and checks that the exact brute force rejects each.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

from oracle import kda_ref

getcontext().prec = 60


# ---------------------------------------------------------------------------
# exact brute force: dense unrolling of the transition products in rationals
# ---------------------------------------------------------------------------

def _exact_exp(x: float) -> Fraction:
    """exp(x) of a binary float to ~60 significant digits, as a Fraction."""
    return Fraction(Decimal(x).exp())


def _mat_mul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    return [[sum((A[i][l] * B[l][j] for l in range(m)), Fraction(0)) for j in range(p)]
            for i in range(n)]


def _eye(n):
    return [[Fraction(int(i == j)) for j in range(n)] for i in range(n)]


def brute_force(q, k, v, g, beta, S0):
    """S_t = Phi(t,0) S0 + sum_{i<=t} Phi(t,i) beta_i k_i v_i^T with
    Phi(t,i) = A_t A_{t-1} ... A_{i+1}, A_s = (I - beta_s k_s k_s^T) Diag(exp g_s);
    o_t = S_t^T q_t. One head; inputs are float arrays [T,Dk] etc.; exact result."""
    T, Dk = q.shape
    Dv = v.shape[1]
    F = lambda x: Fraction(float(x))  # noqa: E731  (binary floats are exact rationals)
    A = []
    for s in range(T):
        a = [_exact_exp(float(g[s, c])) for c in range(Dk)]
        E = [[Fraction(int(i == j)) - F(beta[s]) * F(k[s, i]) * F(k[s, j]) for j in range(Dk)]
             for i in range(Dk)]
        A.append([[E[i][j] * a[j] for j in range(Dk)] for i in range(Dk)])
    writes = [[[F(beta[i]) * F(k[i, r]) * F(v[i, c]) for c in range(Dv)] for r in range(Dk)]
              for i in range(T)]
    S0f = [[F(S0[r, c]) for c in range(Dv)] for r in range(Dk)]
    outs, states = [], []
    for t in range(T):
        # Phi(t, i) for i = t, t-1, ..., -1 built right-to-left
        Phi = _eye(Dk)
        St = [[Fraction(0)] * Dv for _ in range(Dk)]
        for i in range(t, -1, -1):
            Wi = _mat_mul(Phi, writes[i])
            St = [[St[r][c] + Wi[r][c] for c in range(Dv)] for r in range(Dk)]
            Phi = _mat_mul(Phi, A[i])
        P0 = _mat_mul(Phi, S0f)
        St = [[St[r][c] + P0[r][c] for c in range(Dv)] for r in range(Dk)]
        outs.append([sum((St[r][c] * F(q[t, r]) for r in range(Dk)), Fraction(0))
                     for c in range(Dv)])
        states.append(St)
    return (np.array([[float(x) for x in row] for row in outs]),
            np.array([[float(x) for x in row] for row in states[-1]]))


def _tiny_case(seed, T=5, Dk=3, Dv=2, H=2):
    """Small dyadic inputs (exact in float32) with decays exp(g), g float32."""
    rng = np.random.default_rng(seed)
    dy = lambda *s: (rng.integers(-8, 9, size=s) / 8.0).astype(np.float32)  # noqa: E731
    q, k, v = dy(1, T, H, Dk), dy(1, T, H, Dk), dy(1, T, H, Dv)
    g = np.log(rng.choice([0.5, 0.75, 1.0, 0.9], size=(1, T, H, Dk))).astype(np.float32)
    beta = (rng.integers(0, 9, size=(1, T, H)) / 8.0).astype(np.float32)
    S0 = dy(1, H, Dk, Dv)
    return q, k, v, g, beta, S0


def _max_rel(x, ref):
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_P1_bruteforce_exact_numpy(seed):
    q, k, v, g, beta, S0 = _tiny_case(seed)
    o, fin = kda_ref.recurrence(q, k, v, g, beta, initial_state=S0)
    for h in range(q.shape[2]):
        ob, Sb = brute_force(q[0, :, h], k[0, :, h], v[0, :, h], g[0, :, h], beta[0, :, h], S0[0, h])
        assert _max_rel(o[0, :, h], ob) < 1e-13
        assert _max_rel(fin[0, h], Sb) < 1e-13


@pytest.mark.parametrize("seed", [3, 4])
def test_P1_bruteforce_exact_c(oracle_c, seed):
    q, k, v, g, beta, S0 = _tiny_case(seed, T=6, Dk=3, Dv=4)
    o, fin = kda_ref.c_forward(q, k, v, g, beta, initial_state=S0)
    for h in range(q.shape[2]):
        ob, Sb = brute_force(q[0, :, h], k[0, :, h], v[0, :, h], g[0, :, h], beta[0, :, h], S0[0, h])
        assert _max_rel(o[0, :, h], ob) < 1e-13
        assert _max_rel(fin[0, h], Sb) < 1e-13


def test_P2_single_token_closed_form():
    """T=1 expanded: o = (D S0)^T q - beta (k.q) (D S0)^T k + beta (k.q) v; with S0=0, o = beta (k.q) v."""
    rng = np.random.default_rng(7)
    Dk, Dv = 5, 3
    q, k, g = (rng.standard_normal((1, 1, 1, Dk)) for _ in range(3))
    v = rng.standard_normal((1, 1, 1, Dv))
    beta = np.array([[[0.7]]])
    S0 = rng.standard_normal((1, 1, Dk, Dv))
    o, _ = kda_ref.recurrence(q, k, v, g, beta, initial_state=S0)
    DS0 = np.exp(g[0, 0, 0])[:, None] * S0[0, 0]
    kq = float(k[0, 0, 0] @ q[0, 0, 0])
    expect = DS0.T @ q[0, 0, 0] - 0.7 * kq * (DS0.T @ k[0, 0, 0]) + 0.7 * kq * v[0, 0, 0]
    np.testing.assert_allclose(o[0, 0, 0], expect, rtol=1e-13, atol=1e-14)
    o0, _ = kda_ref.recurrence(q, k, v, g, beta)
    np.testing.assert_allclose(o0[0, 0, 0], 0.7 * kq * v[0, 0, 0], rtol=1e-13)


def test_P3_beta_zero_is_pure_decay():
    rng = np.random.default_rng(8)
    B, T, H, Dk, Dv = 1, 37, 2, 6, 4
    q, k = rng.standard_normal((B, T, H, Dk)), rng.standard_normal((B, T, H, Dk))
    v = rng.standard_normal((B, T, H, Dv))
    g = -5.0 / (1 + np.exp(-rng.standard_normal((B, T, H, Dk))))
    S0 = rng.standard_normal((B, H, Dk, Dv))
    beta = np.zeros((B, T, H))
    o, fin = kda_ref.recurrence(q, k, v, g, beta, initial_state=S0)
    Gam = np.cumsum(g[0], axis=0)                                  # [T,H,Dk]
    for t in range(T):
        St = np.exp(Gam[t])[:, :, None] * S0[0]                    # Diag(e^{Gamma_t}) S0
        np.testing.assert_allclose(o[0, t], np.einsum("hk,hkv->hv", q[0, t], St),
                                   rtol=1e-11, atol=1e-300)
    np.testing.assert_allclose(fin[0], np.exp(Gam[-1])[:, :, None] * S0[0], rtol=1e-11)
    o_zero, fin_zero = kda_ref.recurrence(q, k, v, g, beta)
    assert not o_zero.any() and not fin_zero.any()


def test_P4_small_beta_limit_is_gated_linear_attention():
    """With S0 = 0, o_t / beta -> sum_{i<=t} sum_c q_tc exp(Gamma_tc - Gamma_ic) k_ic v_i."""
    rng = np.random.default_rng(9)
    B, T, H, Dk, Dv = 1, 20, 1, 4, 3
    q, k = rng.standard_normal((B, T, H, Dk)), rng.standard_normal((B, T, H, Dk))
    v = rng.standard_normal((B, T, H, Dv))
    g = -1.0 / (1 + np.exp(-rng.standard_normal((B, T, H, Dk))))
    eps = 1e-7
    o, _ = kda_ref.recurrence(q, k, v, g, np.full((B, T, H), eps))
    Gam = np.cumsum(g[0, :, 0], axis=0)
    gla = np.zeros((T, Dv))
    for t in range(T):
        for i in range(t + 1):
            w = float(np.sum(q[0, t, 0] * np.exp(Gam[t] - Gam[i]) * k[0, i, 0]))
            gla[t] += w * v[0, i, 0]
    assert kda_ref.rel_l2(o[0, :, 0] / eps, gla) < 1e-5


def test_P5_orthonormal_keys_rows_evolve_independently():
    """k_t = e_{t}: row s of S only decays, except at step t = s where it becomes
    (1 - beta_t) row + beta_t v_t (after that step's decay)."""
    rng = np.random.default_rng(10)
    Dk, Dv = 6, 5
    T = Dk
    k = np.eye(Dk)[None, :, None, :]                               # [1,T,1,Dk]
    q = rng.standard_normal((1, T, 1, Dk))
    v = rng.standard_normal((1, T, 1, Dv))
    g = -3.0 * rng.random((1, T, 1, Dk))
    beta = rng.random((1, T, 1))
    S0 = rng.standard_normal((1, 1, Dk, Dv))
    _, fin = kda_ref.recurrence(q, k, v, g, beta, initial_state=S0)
    expect = np.zeros((Dk, Dv))
    for s in range(Dk):
        r = S0[0, 0, s].copy()
        for t in range(T):
            r = r * np.exp(g[0, t, 0, s])
            if t == s:
                r = (1 - beta[0, t, 0]) * r + beta[0, t, 0] * v[0, t, 0]
        expect[s] = r
    np.testing.assert_allclose(fin[0, 0], expect, rtol=1e-13, atol=1e-15)
    # g = 0 and beta = 1: the plain delta rule overwrites row t with v_t
    _, fin1 = kda_ref.recurrence(q, k, v, np.zeros_like(g), np.ones_like(beta), initial_state=S0)
    np.testing.assert_allclose(fin1[0, 0], v[0, :, 0], rtol=1e-14)


def test_P6_delta_rule_invariant():
    """beta_t = 1 and |k_t| = 1 give k_t^T S_t = v_t^T for any g and history."""
    rng = np.random.default_rng(11)
    B, T, H, Dk, Dv = 1, 50, 3, 8, 5
    k = rng.standard_normal((B, T, H, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = rng.standard_normal((B, T, H, Dk))
    v = rng.standard_normal((B, T, H, Dv))
    g = -5.0 / (1 + np.exp(-rng.standard_normal((B, T, H, Dk))))
    S0 = rng.standard_normal((B, H, Dk, Dv))
    beta = np.ones((B, T, H))
    for t_end in (1, 17, 50):
        _, fin = kda_ref.recurrence(q[:, :t_end], k[:, :t_end], v[:, :t_end], g[:, :t_end],
                                    beta[:, :t_end], initial_state=S0)
        lhs = np.einsum("hk,hkv->hv", k[0, t_end - 1], fin[0])
        np.testing.assert_allclose(lhs, v[0, t_end - 1], rtol=0, atol=1e-12)


def test_P7_linearity_in_v_and_initial_state():
    rng = np.random.default_rng(12)
    B, T, H, Dk, Dv = 1, 30, 2, 5, 4
    q, k = rng.standard_normal((B, T, H, Dk)), rng.standard_normal((B, T, H, Dk))
    g = -5.0 / (1 + np.exp(-rng.standard_normal((B, T, H, Dk))))
    beta = rng.random((B, T, H))
    v1, v2 = rng.standard_normal((2, B, T, H, Dv))
    s1, s2 = rng.standard_normal((2, B, H, Dk, Dv))
    o1, f1 = kda_ref.recurrence(q, k, v1, g, beta, initial_state=s1)
    o2, f2 = kda_ref.recurrence(q, k, v2, g, beta, initial_state=s2)
    o3, f3 = kda_ref.recurrence(q, k, 2.0 * v1 - 3.0 * v2, g, beta, initial_state=2.0 * s1 - 3.0 * s2)
    np.testing.assert_allclose(o3, 2 * o1 - 3 * o2, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(f3, 2 * f1 - 3 * f2, rtol=1e-10, atol=1e-12)


def test_P8_segment_composition_is_bitwise():
    rng = np.random.default_rng(13)
    B, T, H, Dk, Dv = 1, 41, 2, 4, 3
    q, k = rng.standard_normal((B, T, H, Dk)), rng.standard_normal((B, T, H, Dk))
    v = rng.standard_normal((B, T, H, Dv))
    g = -5.0 / (1 + np.exp(-rng.standard_normal((B, T, H, Dk))))
    beta = rng.random((B, T, H))
    o, fin = kda_ref.recurrence(q, k, v, g, beta)
    T1 = 17
    oa, fa = kda_ref.recurrence(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], beta[:, :T1])
    ob, fb = kda_ref.recurrence(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], beta[:, T1:],
                                initial_state=fa)
    assert np.array_equal(np.concatenate([oa, ob], axis=1), o)
    assert np.array_equal(fb, fin)


def test_packed_sequences_equal_separate_runs(oracle_c):
    rng = np.random.default_rng(14)
    lens = [5, 0, 13, 1, 9]
    T, H, Dk, Dv = sum(lens), 2, 4, 3
    q, k = rng.standard_normal((2, 1, T, H, Dk)).astype(np.float32)
    v = rng.standard_normal((1, T, H, Dv)).astype(np.float32)
    g = (-5.0 / (1 + np.exp(-rng.standard_normal((1, T, H, Dk))))).astype(np.float32)
    beta = rng.random((1, T, H)).astype(np.float32)
    s0 = rng.standard_normal((len(lens), H, Dk, Dv)).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, fin = kda_ref.recurrence(q, k, v, g, beta, initial_state=s0, cu_seqlens=cu)
    oc, finc = kda_ref.c_forward(q, k, v, g, beta, initial_state=s0, cu_seqlens=cu)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        on, fn = kda_ref.recurrence(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b],
                                    initial_state=s0[n:n + 1])
        assert np.array_equal(o[:, a:b], on)
        assert np.array_equal(fin[n], fn[0])
    assert np.array_equal(fin[1], s0[1].astype(np.float64))          # empty sequence keeps S0
    assert kda_ref.rel_l2(oc, o) < 1e-13 and kda_ref.rel_l2(finc, fin) < 1e-13


def test_P9_c_and_numpy_twins_agree(oracle_c):
    rng = np.random.default_rng(15)
    B, T, H, Dk, Dv = 2, 70, 3, 16, 8
    q, k = rng.standard_normal((2, B, T, H, Dk)).astype(np.float32)
    v = rng.standard_normal((B, T, H, Dv)).astype(np.float32)
    g = (-5.0 / (1 + np.exp(-rng.standard_normal((B, T, H, Dk))))).astype(np.float32)
    beta = rng.random((B, T, H)).astype(np.float32)
    s0 = rng.standard_normal((B, H, Dk, Dv)).astype(np.float32)
    o, fin = kda_ref.recurrence(q, k, v, g, beta, initial_state=s0, scale=0.5)
    oc, finc = kda_ref.c_forward(q, k, v, g, beta, initial_state=s0, scale=0.5, nthreads=3)
    assert kda_ref.rel_l2(oc, o) < 1e-13
    assert kda_ref.rel_l2(finc, fin) < 1e-13


def test_decode_step_equals_forward_steps(oracle_c):
    """T single-token decode steps on a cache reproduce the forward over T tokens."""
    rng = np.random.default_rng(16)
    Nb, T, H, Dk, Dv = 3, 9, 2, 8, 4
    q, k = rng.standard_normal((2, Nb, T, H, Dk)).astype(np.float32)
    v = rng.standard_normal((Nb, T, H, Dv)).astype(np.float32)
    g = (-5.0 / (1 + np.exp(-rng.standard_normal((Nb, T, H, Dk))))).astype(np.float32)
    beta = rng.random((Nb, T, H)).astype(np.float32)
    s0 = rng.standard_normal((Nb, H, Dk, Dv)).astype(np.float32)
    o, fin = kda_ref.recurrence(q, k, v, g, beta, initial_state=s0)
    slots = np.array([4, 0, 2])                      # rows -> cache slots (a permutation)
    cache_np = np.zeros((5, H, Dk, Dv))
    cache_np[slots] = s0
    cache_c = cache_np.copy()
    for t in range(T):
        od, cache_np = kda_ref.decode_step(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t],
                                           cache_np, slots)
        oc = kda_ref.c_decode_step(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], cache_c, slots)
        assert np.array_equal(od, o[:, t])
        assert kda_ref.rel_l2(oc, od) < 1e-13
    assert np.array_equal(cache_np[slots], fin)
    assert kda_ref.rel_l2(cache_c[slots], fin) < 1e-13


# ---------------------------------------------------------------------------
# planted mistakes: each wrong variant of the token step must fail brute force
# ---------------------------------------------------------------------------

def _variant_steps():
    def erase_sign(S, q, k, v, g, b, scale=1.0):
        S *= np.exp(g)[:, :, None]
        x = np.einsum("hk,hkv->hv", k, S)
        S += (b[:, None, None] * k[:, :, None]) * (v + x)[:, None, :]
        return scale * np.einsum("hk,hkv->hv", q, S)

    def decay_after_erase(S, q, k, v, g, b, scale=1.0):
        x = np.einsum("hk,hkv->hv", k, S)
        S += (b[:, None, None] * k[:, :, None]) * (v - x)[:, None, :]
        S *= np.exp(g)[:, :, None]
        return scale * np.einsum("hk,hkv->hv", q, S)

    def output_before_update(S, q, k, v, g, b, scale=1.0):
        S *= np.exp(g)[:, :, None]
        out = scale * np.einsum("hk,hkv->hv", q, S)
        x = np.einsum("hk,hkv->hv", k, S)
        S += (b[:, None, None] * k[:, :, None]) * (v - x)[:, None, :]
        return out

    def per_head_decay(S, q, k, v, g, b, scale=1.0):
        S *= np.exp(g.mean(axis=-1))[:, None, None]
        x = np.einsum("hk,hkv->hv", k, S)
        S += (b[:, None, None] * k[:, :, None]) * (v - x)[:, None, :]
        return scale * np.einsum("hk,hkv->hv", q, S)

    def decay_on_value_axis(S, q, k, v, g, b, scale=1.0):
        # decays the d_v axis instead of the d_k axis (only shape-legal when Dk == Dv)
        S *= np.exp(g)[:, None, :]
        x = np.einsum("hk,hkv->hv", k, S)
        S += (b[:, None, None] * k[:, :, None]) * (v - x)[:, None, :]
        return scale * np.einsum("hk,hkv->hv", q, S)

    def dropped_beta_on_erase(S, q, k, v, g, b, scale=1.0):
        S *= np.exp(g)[:, :, None]
        x = np.einsum("hk,hkv->hv", k, S)
        S += k[:, :, None] * (b[:, None] * v - x)[:, None, :]
        return scale * np.einsum("hk,hkv->hv", q, S)

    return dict(erase_sign=erase_sign, decay_after_erase=decay_after_erase,
                output_before_update=output_before_update, per_head_decay=per_head_decay,
                decay_on_value_axis=decay_on_value_axis, dropped_beta_on_erase=dropped_beta_on_erase)


@pytest.mark.parametrize("name", sorted(_variant_steps()))
def test_planted_mistakes_are_caught(monkeypatch, name):
    q, k, v, g, beta, S0 = _tiny_case(21, T=4, Dk=3, Dv=3, H=1)
    ob, Sb = brute_force(q[0, :, 0], k[0, :, 0], v[0, :, 0], g[0, :, 0], beta[0, :, 0], S0[0, 0])
    monkeypatch.setattr(kda_ref, "token_step", _variant_steps()[name])
    o, fin = kda_ref.recurrence(q, k, v, g, beta, initial_state=S0)
    err = max(_max_rel(o[0, :, 0], ob), _max_rel(fin[0, 0], Sb))
    assert err > 1e-6, f"planted mistake {name} was not caught (err={err})"
