"""GPU parity of the intra-sequence split (kda_chunk_fwd_split through the C
ABI) against the fp64 oracle's forward on the same inputs: the split must give
the unsplit recurrence's outputs and final states (bf16 <= 2e-2, fp32 <= 1e-4
relative L2). Cases cover several segment counts, segments longer than the
sequence (empty segments), packed batches with empty and one-token
sequences, weak decay (where the carried state matters most), the fp32
vector-ALU path and the few-head long-sequence shape the split is for.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_chunk_amd as kda
import synth
from tests.gpu_helpers import TOL_BF16, TOL_F32, oracle_chunk, rel, say, to_dev

pytestmark = pytest.mark.gpu


def gpu_split(inp, segments, scale=1.0):
    d = to_dev(inp)
    o, fin = kda.chunk_fwd_split(d["q"], d["k"], d["v"], d["g"], d["beta"], segments,
                                 initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"], scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), fin.cpu().numpy()


def _check(inp, segments, tol, label="", scale=1.0):
    say(f"[case] split {label} segments={segments} q={tuple(inp['q'].shape)} {inp['q'].dtype}")
    o, fin = gpu_split(inp, segments, scale)
    ro, rfin = oracle_chunk(inp, scale=scale)
    eo, ef = rel(o, ro), rel(fin, rfin)
    say(f"        relL2 o={eo:.3e} final={ef:.3e}")
    assert np.isfinite(o).all() and np.isfinite(fin).all()
    assert eo <= tol and ef <= tol, (eo, ef)


@pytest.mark.parametrize("segments", [2, 3, 8])
def test_split_bf16_k3_dims(segments):
    inp = synth.make_chunk_inputs(1, 1000, 3, 128, 128, seed=600 + segments, dtype="bf16", init_state=True)
    _check(inp, segments, TOL_BF16, label="bf16")


@pytest.mark.parametrize("g_mode", ["weak", "zero"])
def test_split_bf16_weak_decay(g_mode):
    # little decay: the state carried across segment boundaries dominates the outputs
    inp = synth.make_chunk_inputs(1, 700, 2, 128, 128, seed=610, dtype="bf16", init_state=True, g_mode=g_mode,
                                  s0_std=0.5)
    _check(inp, 5, TOL_BF16, label=f"bf16 g={g_mode}")


@pytest.mark.parametrize("Dk,Dv,segments", [(64, 32, 4), (128, 128, 3), (16, 64, 6), (32, 16, 2)])
def test_split_f32(Dk, Dv, segments):
    inp = synth.make_chunk_inputs(2, 300, 3, Dk, Dv, seed=620 + Dk + Dv, dtype="f32", init_state=True, s0_std=0.5,
                                  g_mode="weak")
    _check(inp, segments, TOL_F32, label=f"f32 Dk={Dk} Dv={Dv}")


@pytest.mark.parametrize("dtype,tol", [("bf16", TOL_BF16), ("f32", TOL_F32)])
def test_split_packed_ragged(dtype, tol):
    inp = synth.make_chunk_inputs(1, 0, 3, 128, 128, seed=630, dtype=dtype, init_state=True, g_mode="weak",
                                  lengths=[0, 1, 63, 64, 65, 300, 7, 1000])
    _check(inp, 4, tol, label=f"packed {dtype}")


def test_split_bf16_batch_rows_without_initial_state():
    # B > 1 without cu_seqlens (each row a sequence) and zero initial states
    inp = synth.make_chunk_inputs(3, 700, 2, 128, 128, seed=615, dtype="bf16", init_state=False, g_mode="weak")
    _check(inp, 4, TOL_BF16, label="bf16 B=3 no initial state")


def test_split_bf16_scale_and_initial_state():
    # the A pass's outputs carry the scale, so the correction term must too
    inp = synth.make_chunk_inputs(2, 333, 3, 128, 128, seed=617, dtype="bf16", init_state=True, g_mode="weak",
                                  s0_std=0.5)
    _check(inp, 3, TOL_BF16, label="bf16 scale 0.37", scale=0.37)


def test_split_first_segment_rows_equal_the_plain_call():
    """A sequence's first segment starts from its initial state in the split's
    B pass and is computed exactly like the plain call's first rows, so those
    rows agree bit for bit (the later rows carry the correction's rounding)."""
    T, P = 1000, 4
    inp = synth.make_chunk_inputs(2, T, 3, 128, 128, seed=619, dtype="bf16", init_state=True)
    d = to_dev(inp)
    o1, _ = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["initial_state"])
    o2, _ = kda.chunk_fwd_split(d["q"], d["k"], d["v"], d["g"], d["beta"], P, initial_state=d["initial_state"])
    torch.cuda.synchronize()
    seg = -(-T // (P + 1))
    seg = 2 * (-(-seg // 64) * 64)      # first segment: two shares of ceil(T / (P + 1)) rounded up to 64 rows
    say(f"[case] split first segment ({seg} rows of {T}) against the plain call, bitwise")
    assert torch.equal(o1[:, :seg], o2[:, :seg])


def test_split_more_segments_than_chunks():
    inp = synth.make_chunk_inputs(1, 50, 2, 128, 128, seed=640, dtype="bf16", init_state=True, g_mode="weak")
    _check(inp, 8, TOL_BF16, label="T=50")


def test_split_one_segment_is_the_plain_call():
    inp = synth.make_chunk_inputs(1, 300, 4, 128, 128, seed=650, dtype="bf16", init_state=True)
    d = to_dev(inp)
    o1, f1 = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["initial_state"])
    o2, f2 = kda.chunk_fwd_split(d["q"], d["k"], d["v"], d["g"], d["beta"], 1, initial_state=d["initial_state"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_split_is_deterministic():
    inp = synth.make_chunk_inputs(1, 900, 4, 128, 128, seed=660, dtype="bf16", init_state=True)
    a = gpu_split(inp, 4)
    b = gpu_split(inp, 4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.slow
def _every_head(o, fin, ro, rfin, H):
    """relL2 of every head's outputs and final states; returns the worst pair."""
    eo = max(rel(o[:, :, h], ro[:, :, h]) for h in range(H))
    ef = max(rel(fin[:, h], rfin[:, h]) for h in range(H))
    return eo, ef


def test_split_few_heads_long_sequence_every_head():
    # 12 heads (one GPU's share of 96 under head sharding) at T = 32768, S0 ~ N(0, 0.02),
    # 8 segments: every head against the oracle (a head's outputs depend on that head only).
    inp = synth.make_chunk_inputs(1, 32768, 12, 128, 128, seed=670, dtype="bf16", init_state=True)
    say("[case] split H=12 T=32768 segments=8, every head")
    o, fin = gpu_split(inp, 8)
    ro, rfin = oracle_chunk(inp)
    eo, ef = rel(o, ro), rel(fin, rfin)
    wo, wf = _every_head(o, fin, ro, rfin, 12)
    say(f"        relL2 o={eo:.3e} final={ef:.3e}; worst head o={wo:.3e} final={wf:.3e}")
    assert np.isfinite(o).all() and wo <= TOL_BF16 and wf <= TOL_BF16, (wo, wf)


@pytest.mark.slow
def test_split_full_packed_varlen_every_head():
    # The packed workload (16 sequences of U[128, 8192] tokens, H=96) with an initial state, cut into
    # 4 segments per sequence; every head of every sequence against the oracle.
    w = synth.WORKLOADS["k3_varlen16"]
    inp = synth.make_workload(w, init_state=True)
    say(f"[case] split full {w.name} T={inp['q'].shape[1]} segments=4, every head")
    o, fin = gpu_split(inp, 4)
    ro, rfin = oracle_chunk(inp)
    wo, wf = _every_head(o, fin, ro, rfin, 96)
    # every sequence's final state on its own
    ws = max(rel(fin[n], rfin[n]) for n in range(fin.shape[0]))
    say(f"        worst head o={wo:.3e} final={wf:.3e}; worst sequence final={ws:.3e}")
    assert np.isfinite(o).all() and wo <= TOL_BF16 and wf <= TOL_BF16 and ws <= TOL_BF16, (wo, wf, ws)


# --- from raw projections (kda_chunk_fwd_split_prologue) -----------------------

@pytest.mark.parametrize("dtype,Dk,Dv,segments,lengths", [
    ("bf16", 128, 128, 4, None), ("bf16", 128, 128, 3, [300, 0, 1, 517]), ("f32", 64, 32, 3, None),
    ("f32", 128, 128, 5, [200, 333])])
def test_split_prologue_against_oracle(dtype, Dk, Dv, segments, lengths):
    from tests.test_gpu_prologue import oracle_prologue
    inp = synth.make_prologue_inputs(1 if lengths else 2, 0 if lengths else 400, 2, Dk, Dv, seed=630 + segments,
                                     dtype=dtype, init_state=True, lengths=lengths)
    say(f"[case] split from raw projections {dtype} Dk={Dk} Dv={Dv} segments={segments} lengths={lengths}")
    d = to_dev(inp)
    o, fin = kda.chunk_fwd_split_prologue(d["q_raw"], d["k_raw"], d["v"], d["g_logit"], d["beta_logit"], d["A_log"],
                                          d["dt_bias"], segments, initial_state=d["initial_state"],
                                          cu_seqlens=d["cu_seqlens"], scale=0.5)
    o1, fin1 = kda.chunk_fwd_prologue(d["q_raw"], d["k_raw"], d["v"], d["g_logit"], d["beta_logit"], d["A_log"],
                                      d["dt_bias"], initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"],
                                      scale=0.5)
    torch.cuda.synchronize()
    ro, rfin = oracle_prologue(inp, scale=0.5)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    eo, ef = rel(o.float().cpu().numpy(), ro), rel(fin.cpu().numpy(), rfin)
    say(f"        relL2 o={eo:.3e} final={ef:.3e} (unsplit: o={rel(o1.float().cpu().numpy(), ro):.3e})")
    assert eo <= tol and ef <= tol, (eo, ef)
    # one segment is the plain prologue forward
    o2, fin2 = kda.chunk_fwd_split_prologue(d["q_raw"], d["k_raw"], d["v"], d["g_logit"], d["beta_logit"],
                                            d["A_log"], d["dt_bias"], 1, initial_state=d["initial_state"],
                                            cu_seqlens=d["cu_seqlens"], scale=0.5)
    torch.cuda.synchronize()
    assert torch.equal(o2, o1) and torch.equal(fin2, fin1)


def test_split_prologue_gate_bound_below_five_runs_the_float32_passes():
    """bf16, d = 128 with gate_lower_bound = -8: the gate can fall below -5, so
    the split runs its float32 passes (chunk_generic with the prologue)."""
    from tests.test_gpu_prologue import oracle_prologue
    inp = synth.make_prologue_inputs(1, 300, 2, 128, 128, seed=640, dtype="bf16", init_state=True)
    say("[case] split from raw projections, bf16 d=128, gate bound -8")
    d = to_dev(inp)
    o, fin = kda.chunk_fwd_split_prologue(d["q_raw"], d["k_raw"], d["v"], d["g_logit"], d["beta_logit"], d["A_log"],
                                          d["dt_bias"], 3, gate_lower_bound=-8.0, initial_state=d["initial_state"])
    torch.cuda.synchronize()
    ro, rfin = oracle_prologue(inp, lb=-8.0)
    eo, ef = rel(o.float().cpu().numpy(), ro), rel(fin.cpu().numpy(), rfin)
    say(f"        relL2 o={eo:.3e} final={ef:.3e}")
    assert eo <= TOL_BF16 and ef <= TOL_BF16, (eo, ef)
