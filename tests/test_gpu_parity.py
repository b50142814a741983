"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Sizes span several chunks and end in ragged tails; each case checks the whole
output and the final states by relative L2 (fp32 <= 1e-4, bf16 <= 2e-2).
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_chunk_amd as kda
import synth
from oracle import kda_ref
from tests.gpu_helpers import TOL_BF16, TOL_F32, gpu_chunk, oracle_chunk, rel, say, to_dev

pytestmark = pytest.mark.gpu


def _check(inp, tol, chunk=0, scale=1.0, label=""):
    say(f"[case] {label} chunk={chunk} q={tuple(inp['q'].shape)} {inp['q'].dtype}")
    o, fin = gpu_chunk(inp, chunk=chunk, scale=scale)
    ro, rfin = oracle_chunk(inp, scale=scale)
    eo, ef = rel(o, ro), rel(fin, rfin)
    say(f"        relL2 o={eo:.3e} final={ef:.3e}")
    assert np.isfinite(o).all() and np.isfinite(fin).all()
    assert eo <= tol and ef <= tol, (eo, ef)
    return eo, ef


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_tiny_f32_workload(chunk):
    w = synth.WORKLOADS["tiny_f32"]
    _check(synth.make_workload(w), TOL_F32, chunk=chunk, label="tiny_f32")


@pytest.mark.parametrize("Dk,Dv,chunk", [(32, 64, 16), (128, 128, 64), (64, 16, 32), (16, 128, 64)])
def test_f32_general_dims(Dk, Dv, chunk):
    inp = synth.make_chunk_inputs(2, 150, 3, Dk, Dv, seed=100 + Dk + Dv, dtype="f32", init_state=True,
                                  s0_std=0.5)
    _check(inp, TOL_F32, chunk=chunk, label=f"f32 Dk={Dk} Dv={Dv}")


@pytest.mark.parametrize("Dk,Dv", [(16, 16), (128, 16), (16, 128), (64, 32), (128, 64), (32, 128)])
def test_f32_matrix_core_tiles_packed(Dk, Dv):
    """16-row chunks run the float32 products as 16x16 matrix-core tiles: one
    to four column tiles per slice (d_v 16 to 128) and one to eight row tiles
    of the state (d_k 16 to 128), over packed sequences with empty, one-token
    and ragged members and a nonzero initial state."""
    inp = synth.make_chunk_inputs(1, 0, 3, Dk, Dv, seed=520 + Dk + Dv, dtype="f32", init_state=True, s0_std=0.5,
                                  lengths=[1, 0, 47, 16, 33, 80])
    _check(inp, TOL_F32, chunk=16, label=f"f32 tiles Dk={Dk} Dv={Dv}")


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_f32_factored_and_pairwise_grams_mixed(chunk):
    """The float32 kernel forms a chunk's grams from gamma*K and K/gamma while
    every channel's in-chunk cumulative decay stays within e^(+-80), and from
    each pair's own exponential otherwise, chunk by chunk. Here one sequence
    mixes both: mild gates on head 0, gates down to -30 per step on part of
    head 1 followed by no decay at all, single-step drops of -60 on a few
    channels of head 2, the default gates on head 3."""
    inp = synth.make_chunk_inputs(1, 200, 4, 128, 64, seed=510, dtype="f32", init_state=True, s0_std=0.5)
    g = inp["g"].clone()
    g[:, :, 0] *= 0.002
    g[:, 50:120, 1] *= 6.0
    g[:, 120:, 1] = 0.0
    g[:, ::7, 2, :5] = -60.0
    inp["g"] = g
    _check(inp, TOL_F32, chunk=chunk, label="f32 factored and pairwise grams")


@pytest.mark.parametrize("B,T,H", [(1, 293, 5), (3, 200, 16), (2, 64, 8), (1, 1, 3), (3, 77, 96)])
def test_bf16_mfma_path(B, T, H):
    inp = synth.make_chunk_inputs(B, T, H, 128, 128, seed=200 + T + H, dtype="bf16", init_state=True)
    _check(inp, TOL_BF16, label=f"bf16 mfma B={B} T={T} H={H}")


def test_bf16_general_path():
    inp = synth.make_chunk_inputs(1, 170, 4, 64, 64, seed=301, dtype="bf16", init_state=True)
    _check(inp, TOL_BF16, chunk=32, label="bf16 generic 64x64")


@pytest.mark.parametrize("H", [8, 3])
def test_bf16_packed_ragged(H):
    inp = synth.make_chunk_inputs(1, 0, H, 128, 128, seed=400 + H, dtype="bf16", init_state=True,
                                  lengths=[0, 1, 63, 64, 65, 130, 7, 257])
    _check(inp, TOL_BF16, label=f"bf16 packed H={H}")


def test_bf16_packed_many_sequences():
    """More than 256 packed sequences: the matrix-core kernel orders them by
    length within runs of 256 (the last run partial); every sequence must still
    be computed exactly once, so each one's final state is checked on its own."""
    rng = np.random.default_rng(415)
    lengths = [int(x) for x in rng.integers(0, 41, size=600)]
    lengths[0], lengths[300], lengths[599] = 0, 97, 0
    inp = synth.make_chunk_inputs(1, 0, 2, 128, 128, seed=415, dtype="bf16", init_state=True, lengths=lengths)
    _check(inp, TOL_BF16, label="bf16 packed N=600")
    o, fin = gpu_chunk(inp)
    _, rfin = oracle_chunk(inp)
    worst = max(rel(fin[n], rfin[n]) for n in range(len(lengths)))
    say(f"        worst per-sequence final-state relL2 {worst:.3e}")
    assert worst <= TOL_BF16


def test_f32_packed_ragged():
    inp = synth.make_chunk_inputs(1, 0, 2, 32, 32, seed=410, dtype="f32", init_state=True,
                                  lengths=[5, 0, 33, 16])
    _check(inp, TOL_F32, chunk=16, label="f32 packed")


# --- stress variants: distributions where the state paths carry the output ----

@pytest.mark.parametrize("variant", ["weak_decay", "v_zero_s0", "g_zero", "g_bound", "beta_one"])
def test_bf16_stress(variant):
    kw = dict(weak_decay=dict(g_mode="weak"),
              v_zero_s0=dict(v_zero=True, s0_std=1.0),
              g_zero=dict(g_mode="zero"),
              g_bound=dict(g_mode="bound"),
              beta_one=dict(beta_mode="one"))[variant]
    inp = synth.make_chunk_inputs(1, 275, 4, 128, 128, seed=500, dtype="bf16", init_state=True, **kw)
    _check(inp, TOL_BF16, label=f"bf16 stress {variant}")


def test_bf16_first_rows_and_chunk_boundaries():
    """relL2 restricted to the rows right after each chunk boundary (cross-chunk state)."""
    inp = synth.make_chunk_inputs(1, 64 * 5 + 9, 4, 128, 128, seed=510, dtype="bf16", init_state=True,
                                  g_mode="weak")
    o, _ = gpu_chunk(inp)
    ro, _ = oracle_chunk(inp)
    rows = np.concatenate([np.arange(c, c + 4) for c in range(0, 64 * 5 + 9 - 4, 64)])
    e = rel(o[:, rows], ro[:, rows])
    say(f"        boundary rows relL2={e:.3e}")
    assert e <= TOL_BF16


def test_delta_rule_invariant_on_gpu_final_state():
    """beta = 1 with unit-norm fp32 keys: k_T^T S_T = v_T for every head (no oracle involved)."""
    inp = synth.make_chunk_inputs(1, 191, 4, 128, 128, seed=520, dtype="f32", init_state=True,
                                  beta_mode="one")
    _, fin = gpu_chunk(inp)
    kT = inp["k"][0, -1].double().numpy()
    vT = inp["v"][0, -1].double().numpy()
    lhs = np.einsum("hk,hkv->hv", kT, fin[0])
    say(f"        invariant relL2={rel(lhs, vT):.3e}")
    assert rel(lhs, vT) <= TOL_F32


# --- decode step ---------------------------------------------------------------

@pytest.mark.parametrize("dtype,Dk,Dv", [("bf16", 128, 128), ("f32", 128, 128), ("f32", 64, 32), ("bf16", 128, 64),
                                         ("f32", 64, 64)])
def test_recurrent_step_against_oracle(dtype, Dk, Dv):
    say(f"[case] decode {dtype} Dk={Dk} Dv={Dv}")
    Nb, H, n_slots, steps = 6, 3, 9, 5
    cache = synth.make_decode_cache(n_slots, H, Dk, Dv, seed=600)
    slots = torch.tensor([7, 0, 3, 8, 1, 5], dtype=torch.int32)
    dcache = cache.cuda()
    dslots = slots.cuda()
    ref_cache = cache.double().numpy().copy()
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    for step in range(steps):
        x = synth.make_decode_step(Nb, H, Dk, Dv, seed=601, step=step, dtype=dtype)
        d = to_dev(x)
        o = kda.recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], dcache, state_slots=dslots)
        torch.cuda.synchronize()
        ro = kda_ref.c_decode_step(*(x[n].float().numpy() for n in ("q", "k", "v", "g", "beta")),
                                   ref_cache, state_slots=slots.numpy())
        e = rel(o.float().cpu().numpy(), ro)
        say(f"        step {step} relL2 o={e:.3e}")
        assert e <= tol
    ec = rel(dcache.cpu().numpy(), ref_cache)
    say(f"        cache relL2={ec:.3e}")
    assert ec <= tol
    untouched = [s for s in range(n_slots) if s not in slots.tolist()]
    assert torch.equal(dcache.cpu()[untouched], cache[untouched])


# --- properties ---------------------------------------------------------------

def test_bitwise_deterministic():
    inp = synth.make_chunk_inputs(1, 333, 8, 128, 128, seed=700, dtype="bf16", init_state=True)
    o1, f1 = gpu_chunk(inp)
    o2, f2 = gpu_chunk(inp)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


def test_packed_equals_separate_calls_bitwise():
    lens = [70, 0, 129, 64, 5]
    inp = synth.make_chunk_inputs(1, 0, 4, 128, 128, seed=710, dtype="bf16", init_state=True, lengths=lens)
    o, fin = gpu_chunk(inp)
    cu = inp["cu_seqlens"].tolist()
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        if a == b:
            assert np.array_equal(fin[n], inp["initial_state"][n].numpy())
            continue
        part = {x: inp[x][:, a:b] for x in ("q", "k", "v", "g", "beta")}
        part["initial_state"] = inp["initial_state"][n:n + 1]
        part["cu_seqlens"] = None
        on, fn = gpu_chunk(part)
        assert np.array_equal(on, o[:, a:b]) and np.array_equal(fn[0], fin[n])


def test_state_handoff_matches_whole_sequence():
    inp = synth.make_chunk_inputs(1, 320, 4, 128, 128, seed=720, dtype="bf16", init_state=True,
                                  g_mode="weak")
    T1 = 128
    first = {x: inp[x][:, :T1] for x in ("q", "k", "v", "g", "beta")}
    first.update(initial_state=inp["initial_state"], cu_seqlens=None)
    o1, f1 = gpu_chunk(first)
    second = {x: inp[x][:, T1:] for x in ("q", "k", "v", "g", "beta")}
    second.update(initial_state=torch.from_numpy(f1), cu_seqlens=None)
    o2, f2 = gpu_chunk(second)
    ow, fw = gpu_chunk(inp)
    # chunks are aligned at T1 = 2*64, so the split run performs the same arithmetic
    assert np.array_equal(np.concatenate([o1, o2], axis=1), ow)
    assert np.array_equal(f2, fw)


def test_final_state_may_alias_initial_state():
    inp = synth.make_chunk_inputs(1, 130, 4, 128, 128, seed=730, dtype="bf16", init_state=True)
    ref_o, ref_f = gpu_chunk(inp)
    d = to_dev(inp)
    st = d["initial_state"].clone()
    o, fin = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=st,
                           final_state=st)
    torch.cuda.synchronize()
    assert fin.data_ptr() == st.data_ptr()
    assert np.array_equal(o.float().cpu().numpy(), ref_o)
    assert np.array_equal(st.cpu().numpy(), ref_f)


def test_scale_is_linear():
    inp = synth.make_chunk_inputs(1, 100, 4, 128, 128, seed=740, dtype="f32", init_state=True)
    o1, _ = gpu_chunk(inp, scale=1.0)
    o2, _ = gpu_chunk(inp, scale=0.5)
    assert np.array_equal(0.5 * o1, o2)


def test_chunk_size_changes_only_rounding_f32():
    inp = synth.make_chunk_inputs(1, 200, 3, 64, 64, seed=750, dtype="f32", init_state=True)
    o16, f16 = gpu_chunk(inp, chunk=16)
    o64, f64 = gpu_chunk(inp, chunk=64)
    assert rel(o16, o64) < 2e-5 and rel(f16, f64) < 2e-5


def test_decode_steps_reproduce_chunk_forward():
    """T decode steps on a cache equal one chunked forward over the same T tokens."""
    T, H = 70, 4
    inp = synth.make_chunk_inputs(1, T, H, 128, 128, seed=760, dtype="bf16", init_state=True)
    o_chunk, f_chunk = gpu_chunk(inp)
    d = to_dev(inp)
    cache = d["initial_state"].clone()
    outs = []
    for t in range(T):
        outs.append(kda.recurrent_step(d["q"][:, t], d["k"][:, t], d["v"][:, t], d["g"][:, t],
                                       d["beta"][:, t], cache))
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, dim=1).float().cpu().numpy()
    ro, rf = oracle_chunk(inp)
    say(f"        decode vs oracle {rel(o_dec, ro):.3e}, chunk vs oracle {rel(o_chunk, ro):.3e}")
    assert rel(o_dec, ro) <= TOL_BF16 and rel(cache.cpu().numpy(), rf) <= TOL_BF16
    assert rel(o_dec, o_chunk) <= TOL_BF16


def test_zero_length_everything():
    inp = synth.make_chunk_inputs(1, 0, 2, 128, 128, seed=770, dtype="bf16", init_state=True,
                                  lengths=[0, 0, 0])
    o, fin = gpu_chunk(inp)
    assert o.shape == (1, 0, 2, 128)
    assert np.array_equal(fin, inp["initial_state"].numpy())
