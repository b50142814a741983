"""Pins for the oracle's short causal convolution (kernel 4) and its decode step.

The pages give only "a short convolution with kernel size 4 on the query, key
and value projections" (hysenlabs "kimi-k3-mlx", section "Attention is 93
layers split between KDA and a NoPE gated MLA"). The reading pinned here is a
causal depthwise convolution over time, y[t] = sum_i w[:, i] x[t - 3 + i],
with the three inputs before a sequence's start carried in a conv state and an
optional y * sigmoid(y). The pins rest on what that definition fixes by itself
(the impulse response, causality, splitting a sequence with the state handed
over, constant inputs, the sigmoid at ln 3) and catch planted mistakes.
"""
import math

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
IMPLS = [kda_ref.short_conv] + ([kda_ref.c_short_conv] if _c_built() else [])


@pytest.mark.parametrize("conv", IMPLS)
def test_impulse_response_is_the_taps_in_time_order(conv):
    C = 6
    w = np.random.default_rng(0).standard_normal((C, 4)).astype(np.float32)
    x = np.zeros((1, 9, C), dtype=np.float32)
    x[0, 2] = 1.0                                   # impulse at t = 2
    y, _ = conv(x, w)
    w64 = w.astype(np.float64)
    for t in range(9):
        expect = w64[:, 3 - (t - 2)] if 0 <= t - 2 <= 3 else np.zeros(C)
        np.testing.assert_allclose(y[0, t], expect, rtol=0, atol=1e-15)


@pytest.mark.parametrize("conv", IMPLS)
def test_causality(conv):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 20, 5)).astype(np.float32)
    w = rng.standard_normal((5, 4)).astype(np.float32)
    y0, _ = conv(x, w, activation=True)
    x2 = x.copy()
    x2[:, 11] += 1.0
    y1, _ = conv(x2, w, activation=True)
    np.testing.assert_array_equal(y0[:, :11], y1[:, :11])
    assert np.abs(y0[:, 11:15] - y1[:, 11:15]).min() > 0
    np.testing.assert_array_equal(y0[:, 15:], y1[:, 15:])


@pytest.mark.parametrize("conv", IMPLS)
@pytest.mark.parametrize("split", [0, 1, 2, 3, 7])
@pytest.mark.parametrize("act", [False, True])
def test_split_with_state_handoff_equals_one_pass(conv, split, act):
    rng = np.random.default_rng(2 + split)
    x = rng.standard_normal((1, 12, 7)).astype(np.float32)
    w = rng.standard_normal((7, 4)).astype(np.float32)
    s0 = rng.standard_normal((1, 3, 7)).astype(np.float32)
    y, fin = conv(x, w, state=s0, activation=act)
    ya, fa = conv(x[:, :split], w, state=s0, activation=act)
    yb, fb = conv(x[:, split:], w, state=fa.astype(np.float32), activation=act)
    np.testing.assert_array_equal(np.concatenate([ya, yb], axis=1), y)
    np.testing.assert_array_equal(fb, fin)
    # the final state is the last three inputs of the extended sequence
    ext = np.concatenate([s0[0], x[0]], axis=0)
    np.testing.assert_array_equal(fin[0], ext[-3:])


@pytest.mark.parametrize("conv", IMPLS)
def test_constant_input_and_sigmoid_closed_form(conv):
    C = 4
    w = np.array([[0.5, -1.0, 2.0, 0.25]] * C, dtype=np.float32)
    a = np.float32(0.75)
    x = np.full((1, 6, C), a, dtype=np.float32)
    y, _ = conv(x, w)
    np.testing.assert_allclose(y[0, 3:], float(a) * 1.75, rtol=1e-15)      # all taps in range
    np.testing.assert_allclose(y[0, 0], float(a) * 0.25, rtol=1e-15)       # only the last tap (zero state)
    y, _ = conv(x, w, state=np.full((1, 3, C), a, dtype=np.float32))
    np.testing.assert_allclose(y[0], float(a) * 1.75, rtol=1e-15)          # the state fills the window
    # y * sigmoid(y) at y = ln 3 is ln 3 * 3/4
    z = np.float32(math.log(3.0))
    w1 = np.array([[0.0, 0.0, 0.0, 1.0]], dtype=np.float32)
    y, _ = conv(np.full((1, 1, 1), z, dtype=np.float32), w1, activation=True)
    zz = float(z)
    assert abs(y[0, 0, 0] - zz / (1.0 + math.exp(-zz))) < 1e-15
    assert abs(zz / (1.0 + math.exp(-zz)) - math.log(3.0) * 0.75) < 1e-7


@needs_c
def test_c_and_numpy_agree_on_packed_batches():
    rng = np.random.default_rng(3)
    lengths = [0, 1, 2, 3, 5, 17, 40]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T, C = int(cu[-1]), 9
    x = rng.standard_normal((1, T, C)).astype(np.float32)
    w = rng.standard_normal((C, 4)).astype(np.float32)
    st = rng.standard_normal((len(lengths), 3, C)).astype(np.float32)
    for act in (False, True):
        y1, f1 = kda_ref.short_conv(x, w, state=st, cu_seqlens=cu, activation=act)
        y2, f2 = kda_ref.c_short_conv(x, w, state=st, cu_seqlens=cu, activation=act)
        assert np.abs(y1 - y2).max() < 1e-13 and np.abs(f1 - f2).max() == 0.0


@needs_c
def test_decode_steps_reproduce_the_prefill():
    rng = np.random.default_rng(4)
    T, C, Nb = 11, 8, 3
    x = rng.standard_normal((Nb, T, C)).astype(np.float32)
    w = rng.standard_normal((C, 4)).astype(np.float32)
    st = rng.standard_normal((Nb, 3, C)).astype(np.float32)
    y, fin = kda_ref.c_short_conv(x, w, state=st, activation=True)
    cache = st.astype(np.float64).copy()[[2, 0, 1]]           # rows live in permuted slots
    slots = np.array([1, 2, 0])
    for t in range(T):
        yt = kda_ref.c_short_conv_step(x[:, t], w, cache, slots=slots, activation=True)
        np.testing.assert_allclose(yt, y[:, t], rtol=1e-15, atol=1e-15)
    np.testing.assert_array_equal(cache[slots], fin)


def _pins_hold(conv):
    ok = True
    try:
        test_impulse_response_is_the_taps_in_time_order(conv)
        test_constant_input_and_sigmoid_closed_form(conv)
        for split in (1, 7):
            test_split_with_state_handoff_equals_one_pass(conv, split, True)
    except AssertionError:
        ok = False
    return ok


def _mistaken(kind):
    def conv(x, w, state=None, cu_seqlens=None, activation=False):
        x = np.asarray(x, dtype=np.float64)
        w = np.asarray(w, dtype=np.float64)
        if kind == "taps_reversed":
            w = w[:, ::-1]
        B, T, C = x.shape
        y = np.zeros_like(x)
        fin = np.zeros((B, 3, C))
        for b in range(B):
            st = np.zeros((3, C)) if state is None else np.asarray(state, dtype=np.float64)[b]
            if kind == "state_reversed":
                st = st[::-1]
            ext = np.concatenate([st, x[b]], axis=0)
            for t in range(T):
                lo = t - 1 if kind == "window_one_early" else t
                win = ext[lo:lo + 4] if lo >= 0 else np.concatenate([np.zeros((1, C)), ext[:3]])
                acc = (w * win.T).sum(-1)
                if activation:
                    acc = acc * (1.0 / (1.0 + np.exp(-acc)) if kind != "sigmoid_only" else 0.0) + \
                        (1.0 / (1.0 + np.exp(-acc)) if kind == "sigmoid_only" else 0.0)
                y[b, t] = acc
            fin[b] = ext[-3:]
        return y, fin
    return conv


def test_conv_pins_hold_for_the_oracle():
    assert _pins_hold(kda_ref.short_conv)


@pytest.mark.parametrize("kind", ["taps_reversed", "state_reversed", "window_one_early", "sigmoid_only"])
def test_conv_planted_mistakes_are_caught(kind):
    assert not _pins_hold(_mistaken(kind))
