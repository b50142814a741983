"""kda_chunk_fwd_split_static (the split forward on the library's static
scratch, for callers that cannot allocate) against kda_chunk_fwd_split with a
caller workspace: two calls in a row, the second on a smaller input, each
compared bit for bit (the same kernels run on the same inputs; only the
workspace's address differs), plus the first against the fp64 oracle at the
bf16 bar.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_chunk_amd as kda
import synth
from tests.gpu_helpers import TOL_BF16, TOL_F32, oracle_chunk, rel, say, to_dev

pytestmark = pytest.mark.gpu


def _both(inp, segments):
    d = to_dev(inp)
    B, T, H, Dk = d["q"].shape
    Dv = d["v"].shape[-1]
    N = B if d["cu_seqlens"] is None else d["cu_seqlens"].numel() - 1
    ref_o, ref_f = kda.chunk_fwd_split(d["q"], d["k"], d["v"], d["g"], d["beta"], segments,
                                       initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"])
    o = torch.empty((B, T, H, Dv), dtype=d["q"].dtype, device="cuda")
    fin = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device="cuda")
    kda.chunk_fwd_split_static(d["q"], d["k"], d["v"], d["g"], d["beta"], segments,
                               initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"], out=o,
                               final_state=fin)
    torch.cuda.synchronize()
    kda.device_check()
    return o, fin, ref_o, ref_f


def test_static_scratch_matches_workspace_call_twice():
    # call 1: 12 heads at T=8192, 8 segments (44 MB of the 128 MiB scratch)
    inp1 = synth.make_chunk_inputs(1, 8192, 12, 128, 128, seed=950, dtype="bf16", init_state=True)
    need1 = kda.chunk_fwd_split_workspace_bytes(1, 8192, 12, 128, 128, 1, torch.bfloat16, 8)
    say(f"[case] static-scratch split, call 1: B=1 T=8192 H=12 bf16, 8 segments, {need1} bytes of scratch")
    assert need1 <= kda.SPLIT_STATIC_SCRATCH_BYTES
    o, fin, ro, rf = _both(inp1, 8)
    assert torch.equal(o, ro) and torch.equal(fin, rf)
    heads = [0, 11]
    oo, of = oracle_chunk(inp1, heads=heads)
    eo = rel(o.float().cpu().numpy()[:, :, heads], oo)
    ef = rel(fin.cpu().numpy()[:, heads], of)
    say(f"        bit-identical to the workspace call; vs oracle heads {heads}: relL2 o={eo:.3e} final={ef:.3e}")
    assert eo <= TOL_BF16 and ef <= TOL_BF16
    # call 2, right after, smaller: 3 packed fp32 sequences (one empty), 4 heads, d=64, 3 segments
    inp2 = synth.make_chunk_inputs(1, 0, 4, 64, 64, seed=951, dtype="f32", init_state=True,
                                   lengths=[700, 0, 301])
    say("[case] static-scratch split, call 2: packed lengths [700, 0, 301], H=4, d=64, fp32, 3 segments")
    o2, fin2, ro2, rf2 = _both(inp2, 3)
    assert torch.equal(o2, ro2) and torch.equal(fin2, rf2)
    oo2, of2 = oracle_chunk(inp2)
    eo2, ef2 = rel(o2.cpu().numpy(), oo2), rel(fin2.cpu().numpy(), of2)
    say(f"        bit-identical to the workspace call; vs oracle: relL2 o={eo2:.3e} final={ef2:.3e}")
    assert np.isfinite(eo2) and eo2 <= TOL_F32 and ef2 <= TOL_F32
