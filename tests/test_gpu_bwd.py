"""GPU parity of the chunked backward (kda_chunk_bwd through the C ABI) against
the fp64 oracle's reverse-mode gradient (oracle.c_backward) on the same inputs.

The gradients are float32 outputs of float32 arithmetic on inputs that both
sides hold exactly (bf16 inputs are widened without rounding), so every case
uses the float32 bar, relative L2 <= 1e-4, for every gradient tensor.
Cases span several 16-row chunks with ragged tails, every supported head-dim
pair, packed batches with empty and one-token sequences, the gate at its
bound, beta = 1, T = 0, and the full K3 shapes on every head.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_chunk_amd as kda
import synth
from oracle import kda_ref
from tests.gpu_helpers import TOL_F32, rel, say, to_dev

pytestmark = pytest.mark.gpu
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "d_initial")


def gpu_bwd(inp, d_o, d_final, scale=1.0, want_d_initial=True):
    d = to_dev(inp)
    out = kda.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d_o.cuda(),
                        initial_state=d["initial_state"],
                        d_final_state=None if d_final is None else d_final.cuda(),
                        cu_seqlens=d["cu_seqlens"], scale=scale, want_d_initial=want_d_initial)
    torch.cuda.synchronize()
    return [None if x is None else x.cpu().numpy() for x in out]


def oracle_bwd(inp, d_o, d_final, scale=1.0, heads=None):
    f = lambda t: None if t is None else t.float().numpy()  # noqa: E731
    q, k, v, g, beta, s0 = (f(inp[x]) for x in ("q", "k", "v", "g", "beta", "initial_state"))
    do, dfin = f(d_o), f(d_final)
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].numpy().astype(np.int64)
    if heads is not None:
        q, k, v, g, do = (x[:, :, heads] for x in (q, k, v, g, do))
        beta = beta[:, :, heads]
        s0 = None if s0 is None else s0[:, heads]
        dfin = None if dfin is None else dfin[:, heads]
    return kda_ref.c_backward(q, k, v, g, beta, do, initial_state=s0, d_final=dfin, cu_seqlens=cu,
                              scale=scale)


def _check(inp, d_o, d_final, scale=1.0, label="", tol=TOL_F32):
    say(f"[case] bwd {label} q={tuple(inp['q'].shape)} {inp['q'].dtype}")
    got = gpu_bwd(inp, d_o, d_final, scale)
    ref = oracle_bwd(inp, d_o, d_final, scale)
    errs = {}
    for name, x, r in zip(NAMES, got, ref):
        assert np.isfinite(x).all(), name
        errs[name] = rel(x, r) if np.abs(r).max() > 0 else float(np.abs(x).max())
    say("        relL2 " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for name, e in errs.items():
        assert e <= tol, (name, e)
    return got


@pytest.mark.parametrize("Dk,Dv", [(16, 16), (32, 64), (64, 32), (128, 128), (16, 128), (128, 16), (64, 64)])
def test_bwd_f32_dims(Dk, Dv):
    inp = synth.make_chunk_inputs(2, 37, 3, Dk, Dv, seed=500 + Dk + 3 * Dv, dtype="f32", init_state=True,
                                  s0_std=0.5)
    d_o, dfin = synth.make_cotangents(inp, seed=501 + Dk)
    _check(inp, d_o, dfin, scale=0.7, label=f"f32 Dk={Dk} Dv={Dv}")


@pytest.mark.parametrize("B,T,H", [(1, 293, 5), (2, 64, 4), (1, 1, 3), (3, 17, 2)])
def test_bwd_bf16_k3_dims(B, T, H):
    inp = synth.make_chunk_inputs(B, T, H, 128, 128, seed=510 + T + H, dtype="bf16", init_state=True)
    d_o, dfin = synth.make_cotangents(inp, seed=511 + T)
    _check(inp, d_o, dfin, scale=128 ** -0.5, label=f"bf16 B={B} T={T} H={H}")


@pytest.mark.parametrize("dtype,T", [("bf16", 99), ("f32", 50)])
def test_bwd_dv64_one_value_slice(dtype, T):
    # d_k = 128, d_v = 64: the matrix-core backward with one workgroup per
    # (sequence, head) over all value columns (no atomic sums); 7 and 4 chunks
    inp = synth.make_chunk_inputs(2, T, 3, 128, 64, seed=515 + T, dtype=dtype, init_state=True)
    d_o, dfin = synth.make_cotangents(inp, seed=516 + T)
    _check(inp, d_o, dfin, scale=0.5, label=f"{dtype} Dk=128 Dv=64 T={T}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_packed_ragged(dtype):
    inp = synth.make_chunk_inputs(1, 0, 3, 128, 128, seed=520, dtype=dtype, init_state=True,
                                  lengths=[0, 1, 15, 16, 17, 63, 130, 0])
    d_o, dfin = synth.make_cotangents(inp, seed=521)
    _check(inp, d_o, dfin, label=f"packed {dtype}")


def test_bwd_without_state_or_final_cotangent():
    inp = synth.make_chunk_inputs(1, 100, 4, 64, 128, seed=530, dtype="bf16")
    d_o, _ = synth.make_cotangents(inp, seed=531, d_final=False)
    got = _check(inp, d_o, None, label="no S0, no dS_T")
    only = gpu_bwd(inp, d_o, None, want_d_initial=False)
    for a, b in zip(got[:5], only[:5]):
        np.testing.assert_array_equal(a, b)
    assert only[5] is None


@pytest.mark.parametrize("g_mode,beta_mode", [("bound", "default"), ("zero", "one"), ("weak", "zero")])
def test_bwd_gate_and_beta_extremes(g_mode, beta_mode):
    inp = synth.make_chunk_inputs(1, 80, 2, 128, 128, seed=540, dtype="bf16", init_state=True,
                                  g_mode=g_mode, beta_mode=beta_mode)
    d_o, dfin = synth.make_cotangents(inp, seed=541)
    _check(inp, d_o, dfin, label=f"g={g_mode} beta={beta_mode}")


def test_bwd_gate_out_of_range_is_reported():
    """The matrix-core backward (d_k = 128) factors the in-chunk decay and needs
    g in [-5, 0]; a g outside it must be reported by kda_device_check."""
    kda.device_check()
    inp = synth.make_chunk_inputs(1, 200, 2, 128, 128, seed=733, dtype="bf16", init_state=True)
    inp["g"][0, 99, 1, 3] = -6.0
    d_o = torch.randn((1, 200, 2, 128), generator=torch.Generator().manual_seed(733)).to(torch.bfloat16)
    say("[case] bwd d=128 with one g = -6 (token 99, head 1, channel 3)")
    gpu_bwd(inp, d_o, None)
    with pytest.raises(kda.KDAError) as err:
        kda.device_check()
    say(f"        reported: {err.value}")
    assert err.value.status == kda.KDA_ERR_DEVICE and "out of its range" in str(err.value)
    kda.device_check()


def test_bwd_empty_sequence_passes_final_cotangent_through():
    inp = synth.make_chunk_inputs(2, 0, 3, 32, 32, seed=550, dtype="f32", init_state=True)
    d_o, dfin = synth.make_cotangents(inp, seed=551)
    got = gpu_bwd(inp, d_o, dfin)
    np.testing.assert_array_equal(got[5], dfin.numpy())
    got = gpu_bwd(inp, d_o, None)
    np.testing.assert_array_equal(got[5], 0.0)


def test_bwd_is_deterministic():
    inp = synth.make_chunk_inputs(1, 200, 8, 128, 128, seed=560, dtype="bf16", init_state=True)
    d_o, dfin = synth.make_cotangents(inp, seed=561)
    a = gpu_bwd(inp, d_o, dfin)
    b = gpu_bwd(inp, d_o, dfin)
    for name, x, y in zip(NAMES, a, b):
        assert np.array_equal(x, y), name


def _every_head(label, got, ref, H):
    """Every head of every gradient against the oracle (a head's gradients
    depend on that head's inputs only)."""
    for name, x, r in zip(NAMES, got, ref):
        assert np.isfinite(x).all(), name
        worst = (0.0, None)
        for h in range(H):
            e = rel(x[:, h], r[:, h]) if name == "d_initial" else rel(x[:, :, h], r[:, :, h])
            assert e <= TOL_F32, (name, h, e)
            worst = max(worst, (e, h), key=lambda t: t[0])
        say(f"        {label} {name}: whole relL2={rel(x, r):.2e}, worst head {worst[1]} at {worst[0]:.2e}")


@pytest.mark.slow
def test_bwd_full_k3_shape_every_head():
    # B=1, T=4096, H=96, d=128, bf16, every head against the C oracle
    w = synth.WORKLOADS["k3_t4096"]
    inp = synth.make_workload(w)
    d_o, dfin = synth.make_cotangents(inp, seed=570)
    say(f"[case] bwd full {w.name}, every head")
    got = gpu_bwd(inp, d_o, dfin, scale=128 ** -0.5)
    ref = oracle_bwd(inp, d_o, dfin, scale=128 ** -0.5)
    _every_head(w.name, got, ref, w.H)


@pytest.mark.slow
def test_bwd_full_packed_varlen_every_head():
    # The packed workload: 16 sequences of U[128, 8192] tokens, H=96, d=128, bf16, with
    # a final-state cotangent; every head of every sequence against the C oracle.
    w = synth.WORKLOADS["k3_varlen16"]
    inp = synth.make_workload(w)
    d_o, dfin = synth.make_cotangents(inp, seed=580)
    say(f"[case] bwd full {w.name} T={inp['q'].shape[1]}, every head")
    got = gpu_bwd(inp, d_o, dfin, scale=128 ** -0.5)
    ref = oracle_bwd(inp, d_o, dfin, scale=128 ** -0.5)
    _every_head(w.name, got, ref, w.H)
