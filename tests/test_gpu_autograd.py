"""loss.backward() through the autograd entry points (gated_delta_rule_chunk_amd.autograd):
the gradients that reach each input equal the direct backward calls'
(kda_chunk_bwd, kda_chunk_bwd_prologue, kda_chunk_bwd_conv) bit for bit, cast
to the input's dtype; those calls are checked against the oracle elsewhere.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_chunk_amd as kda
import synth
from gated_delta_rule_chunk_amd import autograd as kag
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu

LB, EPS = -5.0, 1e-6


def _leaf(t):
    return None if t is None else t.cuda().requires_grad_(True)


def _weights(shape, seed, dtype=torch.float32):
    rng = np.random.default_rng(seed)
    return torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(dtype).cuda()


@pytest.mark.parametrize("dtype,packed", [("bf16", False), ("f32", True)])
def test_chunk_kda_gradients_equal_the_backward_call(dtype, packed):
    lengths = [40, 0, 77] if packed else None
    inp = synth.make_chunk_inputs(2, 90, 3, 128, 128, seed=1500, dtype=dtype, init_state=True, lengths=lengths)
    say(f"[case] autograd chunk_kda {dtype} packed={packed}")
    x = {n: _leaf(inp[n]) for n in ("q", "k", "v", "g", "beta", "initial_state")}
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].cuda()
    o, fin = kag.chunk_kda(x["q"], x["k"], x["v"], x["g"], x["beta"], initial_state=x["initial_state"],
                           cu_seqlens=cu, scale=0.5)
    Wo, Wf = _weights(o.shape, 1501, o.dtype), _weights(fin.shape, 1502)
    ((o * Wo).float().sum() + (fin * Wf).sum()).backward()
    d = {n: x[n].detach() for n in x}
    ref = kda.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], Wo, initial_state=d["initial_state"],
                        d_final_state=Wf, cu_seqlens=cu, scale=0.5)
    torch.cuda.synchronize()
    for n, r in zip(("q", "k", "v", "g", "beta", "initial_state"), ref):
        assert torch.equal(x[n].grad, r.to(x[n].dtype)), n


def test_chunk_kda_prologue_gradients_equal_the_backward_call():
    inp = synth.make_prologue_inputs(1, 100, 2, 128, 128, seed=1510, dtype="bf16", init_state=True)
    say("[case] autograd chunk_kda_prologue bf16")
    names = ("q_raw", "k_raw", "v", "g_logit", "beta_logit", "A_log", "dt_bias", "initial_state")
    x = {n: _leaf(inp[n]) for n in names}
    o, fin = kag.chunk_kda_prologue(*(x[n] for n in names[:7]), initial_state=x["initial_state"], scale=0.25,
                                    gate_lower_bound=LB, l2_eps=EPS)
    Wo = _weights(o.shape, 1511, o.dtype)
    (o * Wo).float().sum().backward()     # the final state unused: its gradient is zero
    d = {n: x[n].detach() for n in x}
    ref = kda.chunk_bwd_prologue(*(d[n] for n in names[:7]), Wo, gate_lower_bound=LB, l2_eps=EPS,
                                 initial_state=d["initial_state"], d_final_state=torch.zeros_like(fin),
                                 scale=0.25)
    torch.cuda.synchronize()
    for n, r in zip(("q_raw", "k_raw", "v", "g_logit", "beta_logit", "A_log", "dt_bias", "initial_state"), ref):
        assert torch.equal(x[n].grad, r.to(x[n].dtype)), n


def test_chunk_kda_conv_gradients_equal_the_backward_call():
    B, T, H, D = 2, 70, 2, 128
    inp = synth.make_prologue_inputs(B, T, H, D, D, seed=1520, dtype="bf16", init_state=True)
    say("[case] autograd chunk_kda_conv bf16")
    C = H * D
    taps = [_leaf(synth.make_conv_taps(C, 1521, j)) for j in range(3)]
    rng = np.random.default_rng(1522)
    cs = [_leaf(torch.from_numpy(rng.standard_normal((B, 3, C)).astype(np.float32))) for _ in range(3)]
    names = ("q_raw", "k_raw", "v", "g_logit", "beta_logit", "A_log", "dt_bias", "initial_state")
    x = {n: _leaf(inp[n]) for n in names}
    o, fin, conv_fin = kag.chunk_kda_conv(x["q_raw"], x["k_raw"], x["v"], *taps, x["g_logit"], x["beta_logit"],
                                          x["A_log"], x["dt_bias"], conv_states=cs, initial_state=x["initial_state"],
                                          scale=D ** -0.5, gate_lower_bound=LB, l2_eps=EPS)
    Wo, Wf = _weights(o.shape, 1523, o.dtype), _weights(fin.shape, 1524)
    Wc = [_weights(c.shape, 1525 + j) for j, c in enumerate(conv_fin)]
    loss = (o * Wo).float().sum() + (fin * Wf).sum() + sum((c * w).sum() for c, w in zip(conv_fin, Wc))
    loss.backward()
    d = {n: x[n].detach() for n in x}
    ref = kda.chunk_bwd_conv(d["q_raw"], d["k_raw"], d["v"], *(t.detach() for t in taps), d["g_logit"],
                             d["beta_logit"], d["A_log"], d["dt_bias"], Wo, conv_states=[c.detach() for c in cs],
                             d_conv_final=Wc, initial_state=d["initial_state"], d_final_state=Wf, scale=D ** -0.5)
    torch.cuda.synchronize()
    pairs = [(x["q_raw"], "xq"), (x["k_raw"], "xk"), (x["v"], "xv"), (taps[0], "wq"), (taps[1], "wk"),
             (taps[2], "wv"), (cs[0], "conv_state_q"), (cs[1], "conv_state_k"), (cs[2], "conv_state_v"),
             (x["g_logit"], "g_logit"), (x["beta_logit"], "beta_logit"), (x["A_log"], "A_log"),
             (x["dt_bias"], "dt_bias"), (x["initial_state"], "initial_state")]
    for t, n in pairs:
        assert torch.equal(t.grad, ref[n].to(t.dtype)), n


@pytest.mark.parametrize("raw", [False, True])
def test_split_forward_takes_the_same_backward(raw):
    """chunk_kda / chunk_kda_prologue with segments > 1: the split's outputs are
    the unsplit call's within the bf16 bar, and the gradients, which come from
    the saved inputs, equal the unsplit call's bit for bit."""
    from tests.gpu_helpers import TOL_BF16, rel
    say(f"[case] autograd with the split forward, raw={raw}")
    if raw:
        inp = synth.make_prologue_inputs(1, 600, 2, 128, 128, seed=1530, dtype="bf16", init_state=True)
        names = ("q_raw", "k_raw", "v", "g_logit", "beta_logit", "A_log", "dt_bias", "initial_state")
        fn = lambda x, P: kag.chunk_kda_prologue(*(x[n] for n in names[:7]), initial_state=x["initial_state"],  # noqa
                                                 segments=P)
    else:
        inp = synth.make_chunk_inputs(1, 600, 2, 128, 128, seed=1531, dtype="bf16", init_state=True)
        names = ("q", "k", "v", "g", "beta", "initial_state")
        fn = lambda x, P: kag.chunk_kda(*(x[n] for n in names[:5]), initial_state=x["initial_state"], segments=P)  # noqa
    grads, outs = [], []
    for P in (1, 4):
        x = {n: _leaf(inp[n]) for n in names}
        o, fin = fn(x, P)
        Wo, Wf = _weights(o.shape, 1532, o.dtype), _weights(fin.shape, 1533)
        ((o * Wo).float().sum() + (fin * Wf).sum()).backward()
        outs.append((o.detach().float().cpu().numpy(), fin.detach().cpu().numpy()))
        grads.append({n: x[n].grad for n in names})
    torch.cuda.synchronize()
    assert rel(outs[1][0], outs[0][0]) <= TOL_BF16 and rel(outs[1][1], outs[0][1]) <= TOL_BF16
    for n in names:
        assert torch.equal(grads[0][n], grads[1][n]), n
