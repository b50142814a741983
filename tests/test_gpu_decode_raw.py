"""GPU parity of the decode step from raw projections: kda_recurrent_step_prologue
(gate, beta and normalisation prologue + step) and kda_recurrent_step_conv
(short-convolution step + prologue + step), against the fp64 oracle's chain
(convolution step -> prologue -> decode step), over several steps with padding
rows. Bars: relative L2 over whole tensors, fp32 <= 1e-4, bf16 <= 2e-2 (the
forward's); the convolution caches hold copies of the inputs and must match
exactly; the fused convolution call must equal the sequence of standalone
calls bit for bit.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_chunk_amd as kda
import synth
from oracle import kda_ref
from tests.gpu_helpers import TOL_BF16, TOL_F32, rel, say

pytestmark = pytest.mark.gpu

LB, EPS = -5.0, 1e-6
N_SLOTS = 9
# rows 1 and 4 are padding (slot -1, slot past the cache)
SLOTS = [7, -1, 3, 8, N_SLOTS, 0]


def _valid(slots):
    return [r for r, s in enumerate(slots) if 0 <= s < N_SLOTS]


def _oracle_step(raw, conv_out, A_log, dt_bias, ref_cache, slots, scale):
    """The oracle's prologue and decode step on the rows with a slot; conv_out
    (q, k, v) replaces the raw projections when given. Returns o of those rows."""
    rows = _valid(slots)
    qr, kr, vr = conv_out if conv_out is not None else (raw[n].float().numpy()[rows] for n in ("q_raw", "k_raw", "v"))
    gl = raw["g_logit"].float().numpy()[rows]
    bl = raw["beta_logit"].float().numpy()[rows]
    q, k, g, beta = kda_ref.prologue(qr, kr, gl, bl, A_log.numpy(), dt_bias.numpy(), LB, EPS)
    o, new_cache = kda_ref.decode_step(q, k, vr, g, beta, ref_cache, state_slots=[slots[r] for r in rows],
                                       scale=scale)
    return o, new_cache


@pytest.mark.parametrize("dtype,Dk,Dv", [("bf16", 128, 128), ("f32", 128, 128), ("f32", 64, 32),
                                         ("bf16", 16, 128), ("f32", 128, 16), ("bf16", 128, 64)])
def test_step_prologue_against_oracle(dtype, Dk, Dv):
    say(f"[case] decode prologue {dtype} Dk={Dk} Dv={Dv}")
    Nb, H, steps, scale = len(SLOTS), 3, 4, 0.7
    cache = synth.make_decode_cache(N_SLOTS, H, Dk, Dv, seed=700)
    A_log, dt_bias = synth.make_gate_params(H, Dk, seed=701)
    slots = torch.tensor(SLOTS, dtype=torch.int32)
    dcache, dslots = cache.cuda(), slots.cuda()
    dA, db = A_log.cuda(), dt_bias.cuda()
    ref_cache = cache.double().numpy().copy()
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    rows = _valid(SLOTS)
    pad = [r for r in range(Nb) if r not in rows]
    for step in range(steps):
        raw = synth.make_decode_raw_step(Nb, H, Dk, Dv, seed=702, step=step, dtype=dtype)
        if step == 0:
            raw["q_raw"][0, 0] = 0   # a zero row normalises to zero
        d = {n: t.cuda() for n, t in raw.items()}
        o = kda.recurrent_step_prologue(d["q_raw"], d["k_raw"], d["v"], d["g_logit"], d["beta_logit"], dA, db,
                                        dcache, state_slots=dslots, gate_lower_bound=LB, l2_eps=EPS, scale=scale)
        torch.cuda.synchronize()
        ro, ref_cache = _oracle_step(raw, None, A_log, dt_bias, ref_cache, SLOTS, scale)
        og = o.float().cpu().numpy()
        e = rel(og[rows], ro)
        say(f"        step {step} relL2 o={e:.3e}")
        assert e <= tol
        assert not og[pad].any()
    ec = rel(dcache.cpu().numpy(), ref_cache)
    say(f"        cache relL2={ec:.3e}")
    assert ec <= tol
    untouched = [s for s in range(N_SLOTS) if s not in SLOTS]
    assert torch.equal(dcache.cpu()[untouched], cache[untouched])


def _conv_setup(H, Dk, Dv, seed):
    Cs = (H * Dk, H * Dk, H * Dv)
    taps = [synth.make_conv_taps(C, seed, j) for j, C in enumerate(Cs)]
    caches = [synth.make_conv_cache(N_SLOTS, C, seed, j) for j, C in enumerate(Cs)]
    return Cs, taps, caches


@pytest.mark.parametrize("dtype,Dk,Dv,act", [("bf16", 128, 128, True), ("f32", 128, 128, True),
                                             ("f32", 64, 32, False), ("bf16", 32, 64, True)])
def test_step_conv_against_oracle(dtype, Dk, Dv, act):
    say(f"[case] decode conv {dtype} Dk={Dk} Dv={Dv} act={act}")
    Nb, H, steps, scale = len(SLOTS), 3, 5, 1.0
    cache = synth.make_decode_cache(N_SLOTS, H, Dk, Dv, seed=710)
    A_log, dt_bias = synth.make_gate_params(H, Dk, seed=711)
    Cs, taps, caches = _conv_setup(H, Dk, Dv, seed=712)
    slots = torch.tensor(SLOTS, dtype=torch.int32)
    dcache, dslots = cache.cuda(), slots.cuda()
    dA, db = A_log.cuda(), dt_bias.cuda()
    dtaps = [t.cuda() for t in taps]
    dconv = [c.cuda() for c in caches]
    ref_cache = cache.double().numpy().copy()
    ref_conv = [c.double().numpy().copy() for c in caches]
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    rows = _valid(SLOTS)
    rslots = np.array([SLOTS[r] for r in rows], dtype=np.int64)
    pad = [r for r in range(Nb) if r not in rows]
    for step in range(steps):
        raw = synth.make_decode_raw_step(Nb, H, Dk, Dv, seed=713, step=step, dtype=dtype)
        d = {n: t.cuda() for n, t in raw.items()}
        o = kda.recurrent_step_conv(d["q_raw"], d["k_raw"], d["v"], *dtaps, dconv, d["g_logit"], d["beta_logit"],
                                    dA, db, dcache, state_slots=dslots, activation=act, gate_lower_bound=LB,
                                    l2_eps=EPS, scale=scale)
        torch.cuda.synchronize()
        conv_out = []
        for j, name in enumerate(("q_raw", "k_raw", "v")):
            x = raw[name].float().numpy()[rows].reshape(len(rows), Cs[j])
            y = kda_ref.c_short_conv_step(x, taps[j].numpy(), ref_conv[j], slots=rslots, activation=act)
            conv_out.append(y.reshape(raw[name][rows].shape))
        ro, ref_cache = _oracle_step(raw, conv_out, A_log, dt_bias, ref_cache, SLOTS, scale)
        og = o.float().cpu().numpy()
        e = rel(og[rows], ro)
        say(f"        step {step} relL2 o={e:.3e}")
        assert e <= tol
        assert not og[pad].any()
    ec = rel(dcache.cpu().numpy(), ref_cache)
    say(f"        cache relL2={ec:.3e}")
    assert ec <= tol
    for j in range(3):
        np.testing.assert_array_equal(dconv[j].cpu().numpy().astype(np.float64), ref_conv[j])
    untouched = [s for s in range(N_SLOTS) if s not in SLOTS]
    assert torch.equal(dcache.cpu()[untouched], cache[untouched])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_step_conv_equals_the_sequence_of_calls_bitwise(dtype):
    """kda_recurrent_step_conv against kda_short_conv_step x 3 followed by
    kda_recurrent_step_prologue, on copies of the same caches."""
    Nb, H, Dk, Dv, steps = len(SLOTS), 4, 128, 128, 3
    say(f"[case] decode conv == conv steps + prologue step, {dtype}")
    cache = synth.make_decode_cache(N_SLOTS, H, Dk, Dv, seed=720).cuda()
    A_log, dt_bias = (t.cuda() for t in synth.make_gate_params(H, Dk, seed=721))
    Cs, taps, caches = _conv_setup(H, Dk, Dv, seed=722)
    taps = [t.cuda() for t in taps]
    conv_a = [c.cuda() for c in caches]
    conv_b = [c.cuda() for c in caches]
    cache_a, cache_b = cache.clone(), cache.clone()
    slots = torch.tensor(SLOTS, dtype=torch.int32).cuda()
    for step in range(steps):
        raw = {n: t.cuda() for n, t in synth.make_decode_raw_step(Nb, H, Dk, Dv, seed=723, step=step,
                                                                  dtype=dtype).items()}
        oa = kda.recurrent_step_conv(raw["q_raw"], raw["k_raw"], raw["v"], *taps, conv_a, raw["g_logit"],
                                     raw["beta_logit"], A_log, dt_bias, cache_a, state_slots=slots)
        ys = [kda.short_conv_step(raw[n], taps[j], conv_b[j], cache_slots=slots)
              for j, n in enumerate(("q_raw", "k_raw", "v"))]
        ob = kda.recurrent_step_prologue(ys[0], ys[1], ys[2], raw["g_logit"], raw["beta_logit"], A_log, dt_bias,
                                         cache_b, state_slots=slots)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), step
    assert torch.equal(cache_a, cache_b)
    for j in range(3):
        assert torch.equal(conv_a[j], conv_b[j])


def test_decode_conv_steps_reproduce_the_chunk_forward():
    """T tokens through kda_recurrent_step_conv, one at a time from zero
    caches, against kda_chunk_fwd_conv over the same T-token sequences (the
    matrix-core forward with the fused convolution): the same function of
    the inputs, computed two ways."""
    B, T, H, Dk, Dv = 3, 40, 4, 128, 128
    say(f"[case] decode conv x {T} vs chunk forward with convolution, B={B} H={H}")
    inp = synth.make_prologue_inputs(B, T, H, Dk, Dv, seed=730, dtype="bf16")
    Cs, taps, _ = _conv_setup(H, Dk, Dv, seed=731)
    d = {n: (t.cuda() if t is not None else None) for n, t in inp.items()}
    taps = [t.cuda() for t in taps]
    o_ref, fin_ref, _ = kda.chunk_fwd_conv(d["q_raw"], d["k_raw"], d["v"], *taps, d["g_logit"], d["beta_logit"],
                                           d["A_log"], d["dt_bias"], gate_lower_bound=LB, l2_eps=EPS)
    cache = torch.zeros((B, H, Dk, Dv), dtype=torch.float32, device="cuda")
    conv = [torch.zeros((B, 3, C), dtype=torch.float32, device="cuda") for C in Cs]
    outs = []
    for t in range(T):
        step = lambda n: d[n][:, t].contiguous()  # noqa: E731
        outs.append(kda.recurrent_step_conv(step("q_raw"), step("k_raw"), step("v"), *taps, conv, step("g_logit"),
                                            step("beta_logit"), d["A_log"], d["dt_bias"], cache,
                                            gate_lower_bound=LB, l2_eps=EPS))
    torch.cuda.synchronize()
    o = torch.stack(outs, 1)
    eo = rel(o.float().cpu().numpy(), o_ref.float().cpu().numpy())
    ef = rel(cache.cpu().numpy(), fin_ref.cpu().numpy())
    say(f"        relL2 o={eo:.3e} final={ef:.3e}")
    assert eo <= TOL_BF16 and ef <= TOL_BF16


def test_prefill_then_decode_hands_over_every_state():
    """A serving flow: kda_chunk_fwd_conv over a prompt, its final state and
    final conv states written into cache slots, then kda_recurrent_step_conv
    for the following tokens, against kda_chunk_fwd_conv over prompt and
    continuation together. Checks that the prefill's state and conv-state
    layouts are the decode caches' layouts."""
    B, T0, T1, H, D = 3, 50, 6, 4, 128
    say(f"[case] prefill {T0} tokens with kda_chunk_fwd_conv, then {T1} decode steps, B={B}")
    inp = synth.make_prologue_inputs(B, T0 + T1, H, D, D, seed=740, dtype="bf16", init_state=True)
    Cs, taps, _ = _conv_setup(H, D, D, seed=741)
    d = {n: (t.cuda() if t is not None else None) for n, t in inp.items()}
    taps = [t.cuda() for t in taps]
    rng = np.random.default_rng(742)
    s0 = [torch.from_numpy(rng.standard_normal((B, 3, C)).astype(np.float32)).cuda() for C in Cs]
    kw = dict(gate_lower_bound=LB, l2_eps=EPS)
    o_all, fin_all, _ = kda.chunk_fwd_conv(d["q_raw"], d["k_raw"], d["v"], *taps, d["g_logit"], d["beta_logit"],
                                           d["A_log"], d["dt_bias"], conv_states=s0,
                                           initial_state=d["initial_state"], **kw)
    head = {n: d[n][:, :T0].contiguous() for n in ("q_raw", "k_raw", "v", "g_logit", "beta_logit")}
    o_pre, fin_pre, conv_fin = kda.chunk_fwd_conv(head["q_raw"], head["k_raw"], head["v"], *taps, head["g_logit"],
                                                  head["beta_logit"], d["A_log"], d["dt_bias"], conv_states=s0,
                                                  initial_state=d["initial_state"], **kw)
    slots = torch.tensor([5, 0, 2], dtype=torch.int32).cuda()
    n_slots = 7
    cache = torch.zeros((n_slots, H, D, D), dtype=torch.float32, device="cuda")
    cache[slots.long()] = fin_pre
    conv = []
    for j, C in enumerate(Cs):
        c = torch.zeros((n_slots, 3, C), dtype=torch.float32, device="cuda")
        c[slots.long()] = conv_fin[j]
        conv.append(c)
    outs = []
    for t in range(T0, T0 + T1):
        step = lambda n: d[n][:, t].contiguous()  # noqa: E731
        outs.append(kda.recurrent_step_conv(step("q_raw"), step("k_raw"), step("v"), *taps, conv, step("g_logit"),
                                            step("beta_logit"), d["A_log"], d["dt_bias"], cache, state_slots=slots,
                                            **kw))
    torch.cuda.synchronize()
    o = torch.cat([o_pre, torch.stack(outs, 1)], 1)
    eo = rel(o.float().cpu().numpy(), o_all.float().cpu().numpy())
    ef = rel(cache[slots.long()].cpu().numpy(), fin_all.cpu().numpy())
    say(f"        relL2 o={eo:.3e} final={ef:.3e}")
    assert eo <= TOL_BF16 and ef <= TOL_BF16
    # the prompt's outputs are the same call's prefix: equal bit for bit
    assert torch.equal(o_pre, o_all[:, :T0])


def test_decode_step_replays_from_a_captured_graph():
    """A serving loop captures its per-token work in a HIP graph: one
    kda_recurrent_step_conv captured once and replayed for several tokens
    (inputs copied into the captured buffers between replays), against the
    same steps run eagerly on copies of the caches."""
    Nb, H, Dk, Dv, steps = 4, 3, 128, 128, 5
    say(f"[case] decode conv step in a captured graph, {steps} replays")
    cache = synth.make_decode_cache(N_SLOTS, H, Dk, Dv, seed=750).cuda()
    A_log, dt_bias = (t.cuda() for t in synth.make_gate_params(H, Dk, seed=751))
    Cs, taps, caches = _conv_setup(H, Dk, Dv, seed=752)
    taps = [t.cuda() for t in taps]
    slots = torch.tensor([6, -1, 1, 3], dtype=torch.int32).cuda()
    conv_g = [c.cuda() for c in caches]
    conv_e = [c.cuda() for c in caches]
    cache_g, cache_e = cache.clone(), cache.clone()
    raws = [{n: t.cuda() for n, t in synth.make_decode_raw_step(Nb, H, Dk, Dv, seed=753, step=s).items()}
            for s in range(steps)]
    buf = {n: torch.empty_like(t) for n, t in raws[0].items()}
    o_g = torch.empty((Nb, H, Dv), dtype=torch.bfloat16, device="cuda")

    def step(ins, conv, c, out=None):
        return kda.recurrent_step_conv(ins["q_raw"], ins["k_raw"], ins["v"], *taps, conv, ins["g_logit"],
                                       ins["beta_logit"], A_log, dt_bias, c, state_slots=slots, out=out)

    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step(buf, conv_g, cache_g, out=o_g)
    torch.cuda.synchronize()
    for s in range(steps):
        for n in buf:
            buf[n].copy_(raws[s][n])
        graph.replay()
        o_e = step(raws[s], conv_e, cache_e)
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), s
    assert torch.equal(cache_g, cache_e)
    for a, b in zip(conv_g, conv_e):
        assert torch.equal(a, b)
