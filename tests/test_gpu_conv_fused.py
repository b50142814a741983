"""kda_chunk_fwd_conv: the short convolution of q, k and v fused into the chunk
forward from the raw projections.

* Against the unfused GPU sequence (kda_short_conv on q, k and v, outputs
  rounded to the input dtype, then kda_chunk_fwd_prologue): the fused kernel
  convolves in the same arithmetic order and rounds the same way, so o, the
  final state and the final conv states must agree bit for bit.
* Against the oracle's chain (convolution, prologue, recurrence in float64;
  the oracle keeps the convolution's output unrounded): relL2 <= 2e-2 for bf16
  inputs, <= 1e-4 for float32 inputs (the unfused path of other shapes).
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_chunk_amd as kda
import synth
from oracle import kda_ref
from tests.gpu_helpers import TOL_BF16, TOL_F32, rel, say

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _inputs(B, T, H, D, dtype, seed, lengths=None, conv_states=True):
    inp = synth.make_prologue_inputs(B, T, H, D, D, seed=seed, dtype=dtype, init_state=True, lengths=lengths)
    rng = np.random.default_rng(seed + 7)
    C = H * D
    ws = [torch.from_numpy((0.5 * rng.standard_normal((C, 4))).astype(np.float32)) for _ in range(3)]
    N = inp["initial_state"].shape[0]
    s0 = [torch.from_numpy(rng.standard_normal((N, 3, C)).astype(np.float32)) for _ in range(3)] \
        if conv_states else [None, None, None]
    return inp, ws, s0


def _dev(t):
    return None if t is None else t.cuda()


def _fused(inp, ws, s0, act):
    d = {k: _dev(v) for k, v in inp.items()}
    o, fin, cs = kda.chunk_fwd_conv(d["q_raw"], d["k_raw"], d["v"], *(w.cuda() for w in ws), d["g_logit"],
                                    d["beta_logit"], d["A_log"], d["dt_bias"], conv_states=[_dev(s) for s in s0],
                                    activation=act, initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    kda.device_check()
    return o, fin, cs


def _unfused(inp, ws, s0, act):
    d = {k: _dev(v) for k, v in inp.items()}
    ys, fins = [], []
    for name, w, st in zip(("q_raw", "k_raw", "v"), ws, s0):
        y, f = kda.short_conv(d[name], w.cuda(), conv_state=_dev(st), cu_seqlens=d["cu_seqlens"], activation=act)
        ys.append(y)
        fins.append(f)
    o, fin = kda.chunk_fwd_prologue(ys[0], ys[1], ys[2], d["g_logit"], d["beta_logit"], d["A_log"], d["dt_bias"],
                                    initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    return o, fin, fins


def _oracle(inp, ws, s0, act, heads=None):
    B, T, H, D = inp["q_raw"].shape
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].numpy().astype(np.int64)
    hs = list(range(H)) if heads is None else heads
    conv = []
    for name, w, st in zip(("q_raw", "k_raw", "v"), ws, s0):
        x = inp[name].float().numpy()[:, :, hs].reshape(B, T, len(hs) * D)
        wsel = w.numpy().reshape(H, D, 4)[hs].reshape(len(hs) * D, 4)
        ssel = None if st is None else st.numpy().reshape(-1, 3, H, D)[:, :, hs].reshape(-1, 3, len(hs) * D)
        y, _ = kda_ref.c_short_conv(x, wsel, ssel, cu, activation=act)
        conv.append(y.reshape(B, T, len(hs), D))
    return kda_ref.c_prologue_forward(conv[0], conv[1], conv[2], inp["g_logit"].float().numpy()[:, :, hs],
                                      inp["beta_logit"].float().numpy()[:, :, hs], inp["A_log"].numpy(),
                                      inp["dt_bias"].numpy().reshape(H, D)[hs].reshape(-1), -5.0, 1e-6,
                                      initial_state=inp["initial_state"].numpy()[:, hs], cu_seqlens=cu)


CASES = [
    dict(B=1, T=190, H=6, lengths=None, act=True, states=True),
    dict(B=2, T=300, H=4, lengths=None, act=False, states=True),
    dict(B=1, T=0, H=3, lengths=[0, 1, 2, 3, 17, 64, 65, 130, 257], act=True, states=True),
    dict(B=1, T=77, H=96, lengths=None, act=True, states=False),
    # more than 256 packed sequences (the kernel orders them by length within runs of 256)
    dict(B=1, T=0, H=2, lengths=[int(x) for x in np.random.default_rng(77).integers(0, 41, size=300)], act=True,
         states=True),
]


@pytest.mark.parametrize("c", CASES, ids=lambda c: f"B{c['B']}T{c['T']}H{c['H']}"
                         f"L{0 if c['lengths'] is None else len(c['lengths'])}act{int(c['act'])}s{int(c['states'])}")
def test_fused_matches_unfused_bitwise_and_oracle(c):
    inp, ws, s0 = _inputs(c["B"], c["T"], c["H"], 128, "bf16", seed=500 + c["H"] + c["T"], lengths=c["lengths"],
                          conv_states=c["states"])
    say(f"[case] fused conv forward bf16 d=128 {c}")
    o, fin, cs = _fused(inp, ws, s0, c["act"])
    uo, ufin, ucs = _unfused(inp, ws, s0, c["act"])
    assert torch.equal(o, uo), float((o.float() - uo.float()).abs().max())
    assert torch.equal(fin, ufin)
    for a, b in zip(cs, ucs):
        assert torch.equal(a, b)
    ro, rf = _oracle(inp, ws, s0, c["act"])
    eo, ef = rel(o.float().cpu().numpy(), ro), rel(fin.cpu().numpy(), rf)
    say(f"        bit-identical to conv kernels + prologue forward; vs oracle chain relL2 o={eo:.3e} final={ef:.3e}")
    assert eo <= TOL_BF16 and ef <= TOL_BF16


@pytest.mark.parametrize("dtype,D,lb", [("f32", 64, -5.0), ("bf16", 128, -6.0), ("f32", 128, -5.0)])
def test_other_shapes_run_the_convolutions_then_the_forward(dtype, D, lb):
    inp, ws, s0 = _inputs(1, 0, 3, D, dtype, seed=600 + D, lengths=[5, 70, 33])
    say(f"[case] conv forward (unfused path) {dtype} d={D} gate bound {lb}")
    d = {k: _dev(v) for k, v in inp.items()}
    o, fin, _ = kda.chunk_fwd_conv(d["q_raw"], d["k_raw"], d["v"], *(w.cuda() for w in ws), d["g_logit"],
                                   d["beta_logit"], d["A_log"], d["dt_bias"], conv_states=[_dev(s) for s in s0],
                                   activation=True, gate_lower_bound=lb, initial_state=d["initial_state"],
                                   cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    B, T, H, _ = inp["q_raw"].shape
    cu = inp["cu_seqlens"].numpy().astype(np.int64)
    conv = []
    for name, w, st in zip(("q_raw", "k_raw", "v"), ws, s0):
        y, _ = kda_ref.c_short_conv(inp[name].float().numpy().reshape(B, T, H * D), w.numpy(), st.numpy(), cu,
                                    activation=True)
        conv.append(y.reshape(B, T, H, D))
    ro, rf = kda_ref.c_prologue_forward(conv[0], conv[1], conv[2], inp["g_logit"].float().numpy(),
                                        inp["beta_logit"].float().numpy(), inp["A_log"].numpy(),
                                        inp["dt_bias"].numpy(), lb, 1e-6, initial_state=inp["initial_state"].numpy(),
                                        cu_seqlens=cu)
    eo, ef = rel(o.float().cpu().numpy(), ro), rel(fin.cpu().numpy(), rf)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    say(f"        relL2 o={eo:.3e} final={ef:.3e}")
    assert eo <= tol and ef <= tol


@pytest.mark.slow
def test_full_size_k3_t4096():
    w = synth.WORKLOADS["k3_t4096"]
    inp, ws, s0 = _inputs(w.B, w.T, w.H, 128, "bf16", seed=w.seed, conv_states=False)
    say("[case] fused conv forward at full size k3_t4096 (B=1, T=4096, H=96), SiLU")
    o, fin, _ = _fused(inp, ws, s0, True)
    uo, ufin, _ = _unfused(inp, ws, s0, True)
    assert torch.equal(o, uo) and torch.equal(fin, ufin)
    # every head against the oracle's chain
    ro, rf = _oracle(inp, ws, s0, True)
    oh, fh = o.float().cpu().numpy(), fin.cpu().numpy()
    worst = (0.0, None)
    for h in range(w.H):
        eo, ef = rel(oh[:, :, h], ro[:, :, h]), rel(fh[:, h], rf[:, h])
        assert eo <= TOL_BF16 and ef <= TOL_BF16, (h, eo, ef)
        worst = max(worst, (max(eo, ef), h), key=lambda t: t[0])
    say(f"        bit-identical to the unfused sequence; all {w.H} heads vs oracle chain: whole relL2 "
        f"o={rel(oh, ro):.3e} final={rel(fh, rf):.3e}, worst head {worst[1]} at {worst[0]:.3e}")
