"""Explicit failure on the device, and padding rows in the decode calls.

* Bounded waits: the forward's waves hand work to each other through flags
  with bounded waits. A wait that gives up must be reported, never turned into
  silently wrong output (the K3 README's rule that failing paths fail
  explicitly). The give-up is forced from the host with a poll limit of 0, so
  every kernel still runs to its end; kda_device_check must then report
  KDA_ERR_DEVICE, and a following call with the default limit must be clean
  and match the oracle.
* Gate range: the bf16 matrix-core forward needs each 16-row chunk's total
  log-decay in [-84, 0]; a chunk outside it (or a NaN) must be reported by
  kda_device_check, while in-range inputs, the bound itself and the other
  kernels' inputs pass.
* Decode padding: a row whose cache slot is outside [0, n_slots) (-1 here)
  must write a zero output and leave every cache slot it does not own bit for
  bit unchanged; the other rows must equal the oracle run on them alone.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_chunk_amd as kda
import synth
from oracle import kda_ref
from tests.gpu_helpers import TOL_BF16, gpu_chunk, oracle_chunk, rel, say, to_dev

pytestmark = pytest.mark.gpu

DEFAULT_LIMIT = 1 << 22


@pytest.mark.wait_timeout_path
def test_wait_give_up_is_reported():
    kda.device_check()   # nothing pending from earlier tests
    inp = synth.make_chunk_inputs(1, 2048, 96, 128, 128, seed=901, dtype="bf16", init_state=True)
    d = to_dev(inp)
    say("[case] forward with bounded waits forced to give up (poll limit 0), B=1 T=2048 H=96")
    kda.set_wait_limit(0)
    try:
        kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["initial_state"])
        torch.cuda.synchronize()
    finally:
        kda.set_wait_limit(DEFAULT_LIMIT)
    with pytest.raises(kda.KDAError) as err:
        kda.device_check()
    say(f"        reported: {err.value}")
    assert err.value.status == kda.KDA_ERR_DEVICE
    assert "gave up" in str(err.value)
    kda.device_check()   # the report is consumed: a second check is clean
    # the same call with the default limit is clean and correct
    o, fin = gpu_chunk(inp)
    kda.device_check()
    ro, rf = oracle_chunk(inp, heads=[0, 95])
    eo, ef = rel(o[:, :, [0, 95]], ro), rel(fin[:, [0, 95]], rf)
    say(f"        default limit: relL2 o={eo:.3e} final={ef:.3e}")
    assert eo <= TOL_BF16 and ef <= TOL_BF16


@pytest.mark.parametrize("case", ["deep", "positive", "nan"])
def test_gate_out_of_range_is_reported(case):
    """The bf16 matrix-core forward needs each 16-row chunk's total log-decay
    per channel in [-84, 0]: one g of -90, a chunk whose sum is positive, or a
    NaN must be reported by kda_device_check."""
    kda.device_check()
    inp = synth.make_chunk_inputs(1, 300, 4, 128, 128, seed=905, dtype="bf16", init_state=True, g_mode="weak")
    inp["g"][0, 157, 2, 77] = {"deep": -90.0, "positive": 1.0, "nan": float("nan")}[case]
    d = to_dev(inp)
    say(f"[case] bf16 d=128 forward with one g out of range ({case}; token 157, head 2, channel 77)")
    kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["initial_state"])
    with pytest.raises(kda.KDAError) as err:
        kda.device_check()
    say(f"        reported: {err.value}")
    assert err.value.status == kda.KDA_ERR_DEVICE and "out of its range" in str(err.value)
    kda.device_check()   # consumed


def test_gate_in_range_passes():
    kda.device_check()
    # g exactly -5 on 64 rows (chunk totals of -80) and 0 on 16 rows
    inp = synth.make_chunk_inputs(1, 300, 4, 128, 128, seed=906, dtype="bf16", init_state=True)
    inp["g"][0, :64] = -5.0
    inp["g"][0, 64:80] = 0.0
    # one g below -5 whose chunk total stays far from -84: computed exactly, not reported
    inp["g"][0, 200, 1, 9] = -5.25
    o, fin = gpu_chunk(inp)
    kda.device_check()
    ro, rf = oracle_chunk(inp)
    eo, ef = rel(o, ro), rel(fin, rf)
    say(f"        in-range gates: relL2 o={eo:.3e} final={ef:.3e}")
    assert eo <= TOL_BF16 and ef <= TOL_BF16
    # the float32 kernel takes any finite g
    inp32 = synth.make_chunk_inputs(1, 100, 2, 64, 64, seed=907, dtype="f32", init_state=True)
    inp32["g"][0, 10, 1, 5] = -90.0
    gpu_chunk(inp32, chunk=16)
    kda.device_check()


@pytest.mark.wait_timeout_path
def test_wait_give_up_is_reported_prologue():
    kda.device_check()
    inp = synth.make_prologue_inputs(1, 2048, 96, 128, 128, seed=902, dtype="bf16")
    d = to_dev(inp)
    say("[case] prologue forward with bounded waits forced to give up (poll limit 0), B=1 T=2048 H=96")
    kda.set_wait_limit(0)
    try:
        kda.chunk_fwd_prologue(d["q_raw"], d["k_raw"], d["v"], d["g_logit"], d["beta_logit"], d["A_log"],
                               d["dt_bias"])
        torch.cuda.synchronize()
    finally:
        kda.set_wait_limit(DEFAULT_LIMIT)
    with pytest.raises(kda.KDAError) as err:
        kda.device_check()
    assert err.value.status == kda.KDA_ERR_DEVICE
    kda.device_check()


def test_decode_padding_slots():
    Nb, H, D, n_slots = 5, 4, 128, 6
    slots = [2, -1, 5, 6, 0]          # rows 1 and 3 are padding (-1, and n_slots itself)
    cache = synth.make_decode_cache(n_slots, H, D, D, seed=903)
    x = synth.make_decode_step(Nb, H, D, D, seed=903, step=0)
    say(f"[case] decode with padding slots {slots}, n_slots={n_slots}")
    dc = cache.cuda()
    dx = to_dev(x)
    o = kda.recurrent_step(dx["q"], dx["k"], dx["v"], dx["g"], dx["beta"], dc,
                           state_slots=torch.tensor(slots, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    o = o.float().cpu()
    after = dc.cpu()
    valid = [r for r, s in enumerate(slots) if 0 <= s < n_slots]
    ref_cache = cache.double().numpy().copy()
    f = lambda t: t[valid].float().numpy()  # noqa: E731
    ro = kda_ref.c_decode_step(*(f(x[n]) for n in ("q", "k", "v", "g", "beta")), ref_cache,
                               state_slots=[slots[r] for r in valid])
    assert torch.equal(o[[1, 3]], torch.zeros_like(o[[1, 3]]))
    for s in (1, 3, 4):
        assert torch.equal(after[s], cache[s]), f"slot {s} must be untouched"
    eo = rel(o[valid].numpy(), ro)
    ec = rel(after.numpy(), ref_cache)
    say(f"        relL2 o={eo:.3e} cache={ec:.3e}")
    assert eo <= TOL_BF16 and ec <= TOL_BF16


def test_conv_step_padding_slots():
    Nb, C, n_slots = 4, 256, 5
    slots = [3, -1, 0, 7]
    rng = np.random.default_rng(904)
    x = torch.from_numpy(rng.standard_normal((Nb, C)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((0.5 * rng.standard_normal((C, 4))).astype(np.float32))
    cache = torch.from_numpy(rng.standard_normal((n_slots, 3, C)).astype(np.float32))
    say(f"[case] conv decode step with padding slots {slots}, n_slots={n_slots}")
    dc = cache.cuda()
    y = kda.short_conv_step(x.cuda(), w.cuda(), dc, cache_slots=torch.tensor(slots, dtype=torch.int32,
                                                                             device="cuda"), activation=True)
    torch.cuda.synchronize()
    y = y.float().cpu()
    after = dc.cpu()
    assert torch.equal(y[[1, 3]], torch.zeros_like(y[[1, 3]]))
    for s in (1, 2, 4):
        assert torch.equal(after[s], cache[s]), f"slot {s} must be untouched"
    valid = [0, 2]
    ref_cache = cache.double().numpy().copy()
    ry = kda_ref.c_short_conv_step(x[valid].float().numpy(), w.numpy(), ref_cache,
                                   slots=[slots[r] for r in valid], activation=True)
    ey = rel(y[valid].numpy(), ry)
    say(f"        relL2 y={ey:.3e}")
    assert ey <= TOL_BF16
    assert rel(after.numpy(), ref_cache) <= 1e-7   # the cache holds copies of inputs
