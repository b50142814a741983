"""GPU parity on tensors larger than 2 GiB, where a 32-bit byte or element
offset would wrap: the bf16 chunk forward (unsplit and split into segments)
and backward at B=1, T=90000, H=96
(2.2 GB per q/k/v/g/o tensor, 4.4 GB per fp32 gradient, 35 GB of backward
workspace, a ragged 16-row tail), the short convolution at the same T over
C=12288 channels, and the decode step on a 2.5 GB state cache.

Heads, the channels of the convolution and the cache slots are independent.
So only sampled heads (channels, slots) hold seeded inputs and the rest stay zero, and the fp64
oracle recomputes exactly those units in full. A unit that read another
unit's bytes (a wrapped offset) would see zeros or foreign data and miss the
bar, and the zero units must come out exactly zero. Bars as for the full-size
tests: relL2 <= 2e-2 for the bf16 forward and convolution, 1e-4 for the
backward (both sides differentiate the same bf16 values).
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_chunk_amd as kda
import synth
from oracle import kda_ref
from tests.gpu_helpers import TOL_BF16, TOL_F32, rel, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

T_BIG = 90000           # 90000 * 96 * 256 B = 2.21e9 B > 2^31 per tensor
H_BIG = 96
HEADS = [0, 95]         # the first and the last head: both cross 2^31 after token 87382
C_BIG = 96 * 128
CHANNELS = list(range(0, 8)) + list(range(C_BIG - 8, C_BIG))


def _f(t):
    return t.float().numpy()


def _spread(small, dev):
    """Full-size device inputs whose heads HEADS hold the sampled inputs."""
    full = {}
    for name in ("q", "k", "v", "g"):
        t = torch.zeros((1, T_BIG, H_BIG, 128), dtype=torch.bfloat16, device=dev)
        t[:, :, HEADS] = small[name].to(dev)
        full[name] = t
    full["beta"] = torch.zeros((1, T_BIG, H_BIG), dtype=torch.bfloat16, device=dev)
    full["beta"][:, :, HEADS] = small["beta"].to(dev)
    return full


@pytest.mark.parametrize("segments", [1, 4])
def test_forward_beyond_2gib(segments):
    say(f"[case] forward B=1 T={T_BIG} H={H_BIG} heads {HEADS} (tensors of {T_BIG * H_BIG * 256 / 1e9:.2f} GB), "
        f"{'unsplit' if segments == 1 else f'{segments} segments'}")
    small = synth.make_chunk_inputs(1, T_BIG, len(HEADS), 128, 128, seed=2024, dtype="bf16")
    full = _spread(small, "cuda")
    if segments == 1:
        o, fin = kda.chunk_fwd(full["q"], full["k"], full["v"], full["g"], full["beta"])
    else:
        o, fin = kda.chunk_fwd_split(full["q"], full["k"], full["v"], full["g"], full["beta"], segments)
    torch.cuda.synchronize()
    o_s = o[:, :, HEADS].float().cpu().numpy()
    f_s = fin[:, HEADS].cpu().numpy()
    # the zero heads must stay exactly zero (a wrapped store would land there)
    zero_heads = [h for h in range(H_BIG) if h not in HEADS]
    assert float(o[:, :, zero_heads].abs().amax()) == 0.0
    assert float(fin[:, zero_heads].abs().amax()) == 0.0
    del o, fin, full
    torch.cuda.empty_cache()
    ro, rf = kda_ref.c_forward(_f(small["q"]), _f(small["k"]), _f(small["v"]), _f(small["g"]),
                               _f(small["beta"]))
    eo, ef = rel(o_s, ro), rel(f_s, rf)
    e_tail = rel(o_s[:, -100:], ro[:, -100:])
    say(f"        relL2 o={eo:.3e} final={ef:.3e} last100={e_tail:.3e}")
    assert eo <= TOL_BF16 and ef <= TOL_BF16 and e_tail <= TOL_BF16, (eo, ef, e_tail)


def test_backward_beyond_2gib():
    say(f"[case] backward B=1 T={T_BIG} H={H_BIG} heads {HEADS}")
    small = synth.make_chunk_inputs(1, T_BIG, len(HEADS), 128, 128, seed=2025, dtype="bf16")
    d_o_s, dfin_s = synth.make_cotangents(small, seed=2026)
    dev = "cuda"
    full = _spread(small, dev)
    d_o = torch.zeros((1, T_BIG, H_BIG, 128), dtype=torch.bfloat16, device=dev)
    d_o[:, :, HEADS] = d_o_s.to(dev)
    dfin = torch.zeros((1, H_BIG, 128, 128), dtype=torch.float32, device=dev)
    dfin[:, HEADS] = dfin_s.to(dev)
    scale = 128 ** -0.5
    got = kda.chunk_bwd(full["q"], full["k"], full["v"], full["g"], full["beta"], d_o, d_final_state=dfin,
                        scale=scale, want_d_initial=True)
    torch.cuda.synchronize()
    zero_heads = [h for h in range(H_BIG) if h not in HEADS]
    sampled = []
    for name, x in zip(("dq", "dk", "dv", "dg", "dbeta", "d_initial"), got):
        sel = (slice(None), HEADS) if name == "d_initial" else (slice(None), slice(None), HEADS)
        zsel = (slice(None), zero_heads) if name == "d_initial" else (slice(None), slice(None), zero_heads)
        assert bool(torch.isfinite(x[sel]).all()), name
        assert float(x[zsel].abs().amax()) == 0.0, name
        sampled.append((name, x[sel].cpu().numpy()))
    del got, full, d_o, dfin
    torch.cuda.empty_cache()
    ref = kda_ref.c_backward(_f(small["q"]), _f(small["k"]), _f(small["v"]), _f(small["g"]), _f(small["beta"]),
                             _f(d_o_s), initial_state=None, d_final=dfin_s.float().numpy(), cu_seqlens=None,
                             scale=scale)
    errs = {name: rel(x, r) for (name, x), r in zip(sampled, ref)}
    say("        relL2 " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for name, e in errs.items():
        assert e <= TOL_F32, (name, e)


def test_short_conv_beyond_2gib():
    say(f"[case] short conv B=1 T={T_BIG} C={C_BIG} channels {CHANNELS[0]}..{CHANNELS[7]}, "
        f"{CHANNELS[8]}..{CHANNELS[-1]} (x of {T_BIG * C_BIG * 2 / 1e9:.2f} GB)")
    rng = np.random.default_rng(4049)
    xs = torch.from_numpy(rng.standard_normal((1, T_BIG, len(CHANNELS))).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((0.5 * rng.standard_normal((C_BIG, 4))).astype(np.float32))
    s0 = torch.from_numpy(rng.standard_normal((1, 3, C_BIG)).astype(np.float32))
    dev = "cuda"
    x = torch.zeros((1, T_BIG, C_BIG), dtype=torch.bfloat16, device=dev)
    x[:, :, CHANNELS] = xs.to(dev)
    y, fin = kda.short_conv(x, w.to(dev), conv_state=s0.to(dev), activation=True)
    torch.cuda.synchronize()
    y_s = y[:, :, CHANNELS].float().cpu().numpy()
    f_s = fin[:, :, CHANNELS].cpu().numpy()
    del x, y, fin
    ry, rfin = kda_ref.c_short_conv(xs.float().numpy(), w[CHANNELS].contiguous().numpy(),
                                    s0[:, :, CHANNELS].contiguous().numpy(), None, activation=True)
    ey, ef = rel(y_s, ry), rel(f_s, rfin)
    e_tail = rel(y_s[:, -100:], ry[:, -100:])
    say(f"        relL2 y={ey:.3e} final={ef:.3e} last100={e_tail:.3e}")
    assert ey <= TOL_BF16 and e_tail <= TOL_BF16 and ef <= 1e-7, (ey, ef, e_tail)


def test_decode_step_cache_beyond_2gib():
    n_slots = 400          # 400 * 96 * 64 KiB = 2.5 GB of fp32 state cache
    slots = [399, 0, 350, 200]
    say(f"[case] decode step, cache [{n_slots},{H_BIG},128,128] fp32 ({n_slots * H_BIG * 65536 / 1e9:.2f} GB), "
        f"slots {slots}")
    small = synth.make_decode_cache(len(slots), H_BIG, 128, 128, seed=2027)
    dev = "cuda"
    cache = torch.zeros((n_slots, H_BIG, 128, 128), dtype=torch.float32, device=dev)
    cache[slots] = small.to(dev)
    dslots = torch.tensor(slots, dtype=torch.int32, device=dev)
    ref_cache = small.double().numpy().copy()
    for step in range(2):
        x = synth.make_decode_step(len(slots), H_BIG, 128, 128, seed=2028, step=step, dtype="bf16")
        d = {n: x[n].to(dev) for n in ("q", "k", "v", "g", "beta")}
        o = kda.recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], cache, state_slots=dslots)
        torch.cuda.synchronize()
        ro = kda_ref.c_decode_step(*(_f(x[n]) for n in ("q", "k", "v", "g", "beta")), ref_cache,
                                   state_slots=np.arange(len(slots), dtype=np.int32))
        e = rel(o.float().cpu().numpy(), ro)
        say(f"        step {step} relL2 o={e:.3e}")
        assert e <= TOL_BF16
    ec = rel(cache[slots].cpu().numpy(), ref_cache)
    untouched = [s for s in range(n_slots) if s not in slots]
    say(f"        cache relL2={ec:.3e}")
    assert ec <= TOL_BF16
    assert float(cache[untouched].abs().amax()) == 0.0
