"""GPU parity of the short causal convolution (kda_short_conv and its decode
step) against the fp64 oracle, and of the chain convolution -> fused-prologue
forward against the oracle's chain. Bars: relative L2 over whole tensors,
fp32 <= 1e-4, bf16 <= 2e-2 (the forward's); the decode steps must reproduce
the GPU prefill bit for bit.
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


def _inputs(B, T, C, dtype, seed, lengths=None, state=True):
    rng = np.random.default_rng(seed)
    cu = None
    if lengths is not None:
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        B, T = 1, int(cu[-1])
    N = B if cu is None else len(lengths)
    x = torch.from_numpy(rng.standard_normal((B, T, C)).astype(np.float32)).to(DT[dtype])
    w = torch.from_numpy((0.5 * rng.standard_normal((C, 4))).astype(np.float32))
    s0 = torch.from_numpy(rng.standard_normal((N, 3, C)).astype(np.float32)) if state else None
    return x, w, s0, (None if cu is None else torch.from_numpy(cu))


def _check(x, w, s0, cu, act, tol, label):
    say(f"[case] conv {label} x={tuple(x.shape)} {x.dtype} act={act} state={s0 is not None}")
    dev = "cuda"
    y, fin = kda.short_conv(x.to(dev), w.to(dev), conv_state=None if s0 is None else s0.to(dev),
                            cu_seqlens=None if cu is None else cu.to(dev), activation=act)
    torch.cuda.synchronize()
    ry, rfin = kda_ref.c_short_conv(x.float().numpy(), w.numpy(), None if s0 is None else s0.numpy(),
                                    None if cu is None else cu.numpy().astype(np.int64), activation=act)
    ey, ef = rel(y.float().cpu().numpy(), ry), rel(fin.cpu().numpy(), rfin)
    say(f"        relL2 y={ey:.3e} final={ef:.3e}")
    assert ey <= tol and ef <= 1e-7, (ey, ef)      # the final state copies inputs exactly


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("act", [True, False])
@pytest.mark.parametrize("B,T,C", [(2, 150, 256), (1, 33, 12288), (3, 5, 64)])
def test_prefill(dtype, act, B, T, C):
    x, w, s0, cu = _inputs(B, T, C, dtype, seed=B * 1000 + T + C)
    _check(x, w, s0, cu, act, TOL_BF16 if dtype == "bf16" else TOL_F32, f"B={B} T={T} C={C}")


@pytest.mark.parametrize("state", [True, False])
def test_packed_ragged(state):
    x, w, s0, cu = _inputs(1, 0, 384, "bf16", seed=77, lengths=[0, 1, 2, 3, 17, 0, 40, 16, 33], state=state)
    _check(x, w, s0, cu, True, TOL_BF16, "packed")


def test_final_state_may_alias_initial_state():
    x, w, s0, cu = _inputs(1, 0, 128, "f32", seed=78, lengths=[1, 2, 5])
    dev = "cuda"
    st = s0.to(dev).clone()
    _, fin = kda.short_conv(x.to(dev), w.to(dev), conv_state=st, cu_seqlens=cu.to(dev), final_state=st)
    torch.cuda.synchronize()
    _, rfin = kda_ref.c_short_conv(x.numpy(), w.numpy(), s0.numpy(), cu.numpy().astype(np.int64), activation=True)
    assert fin.data_ptr() == st.data_ptr()
    np.testing.assert_array_equal(st.cpu().numpy(), rfin.astype(np.float32))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_steps_reproduce_the_prefill(dtype):
    Nb, T, C = 5, 9, 512
    x, w, s0, _ = _inputs(Nb, T, C, dtype, seed=79)
    dev = "cuda"
    y, fin = kda.short_conv(x.to(dev), w.to(dev), conv_state=s0.to(dev), activation=True)
    slots = torch.tensor([3, 0, 6, 1, 4], dtype=torch.int32)
    cache = torch.zeros((7, 3, C), dtype=torch.float32)
    cache[slots.long()] = s0
    cache = cache.to(dev)
    ys = []
    for t in range(T):
        ys.append(kda.short_conv_step(x[:, t].contiguous().to(dev), w.to(dev), cache, cache_slots=slots.to(dev)))
    torch.cuda.synchronize()
    say(f"[case] conv decode {dtype}: {T} steps of {Nb} rows")
    np.testing.assert_array_equal(torch.stack(ys, 1).float().cpu().numpy(), y.float().cpu().numpy())
    np.testing.assert_array_equal(cache.cpu().numpy()[slots.long().numpy()], fin.cpu().numpy())


def test_conv_then_prologue_forward_chain():
    """q, k, v through the convolution (SiLU), then the fused-prologue forward,
    against the oracle's convolution and prologue forward in float64."""
    B, T, H, D = 1, 190, 6, 128
    inp = synth.make_prologue_inputs(B, T, H, D, D, seed=1234, dtype="bf16", init_state=True)
    rng = np.random.default_rng(99)
    ws = [torch.from_numpy((0.5 * rng.standard_normal((H * D, 4))).astype(np.float32)) for _ in range(3)]
    dev = "cuda"
    conv = {}
    ref_conv = {}
    for name, w in zip(("q_raw", "k_raw", "v"), ws):
        y, _ = kda.short_conv(inp[name].to(dev), w.to(dev), activation=True, output_final_state=False)
        conv[name] = y
        ry, _ = kda_ref.c_short_conv(inp[name].float().numpy().reshape(B, T, H * D), w.numpy(), activation=True)
        ref_conv[name] = ry.reshape(B, T, H, D)
    o, fin = kda.chunk_fwd_prologue(conv["q_raw"], conv["k_raw"], conv["v"], inp["g_logit"].to(dev),
                                    inp["beta_logit"].to(dev), inp["A_log"].to(dev), inp["dt_bias"].to(dev),
                                    initial_state=inp["initial_state"].to(dev))
    torch.cuda.synchronize()
    ro, rfin = kda_ref.c_prologue_forward(ref_conv["q_raw"], ref_conv["k_raw"], ref_conv["v"],
                                          inp["g_logit"].float().numpy(), inp["beta_logit"].float().numpy(),
                                          inp["A_log"].numpy(), inp["dt_bias"].numpy(), -5.0, 1e-6,
                                          initial_state=inp["initial_state"].numpy())
    # (the oracle's chain keeps the convolution's output in float64; the GPU
    # rounds it to bf16 before the forward)
    eo, ef = rel(o.float().cpu().numpy(), ro), rel(fin.cpu().numpy(), rfin)
    say(f"[case] conv -> prologue forward: relL2 o={eo:.3e} final={ef:.3e}")
    assert eo <= TOL_BF16 and ef <= TOL_BF16, (eo, ef)
