"""Host checks of the seeded input generator against the facts the pages print."""
import json
import os

import numpy as np
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "k3_kda_facts.json")


def test_workload_shapes_match_the_pages():
    facts = json.load(open(GOLDEN))
    assert synth.K3_HEADS == facts["num_heads"]["value"]
    assert synth.K3_HEAD_DIM == facts["head_dim"]["value"]
    assert synth.GATE_LOWER_BOUND == facts["gate_lower_bound"]["value"]
    assert facts["a_log_len"]["value"] * facts["num_heads"]["value"] == facts["a_log_len"]["dt_bias_len"]
    for name in ("k3_t4096", "k3_t32768_s0", "k3_varlen16"):
        w = synth.WORKLOADS[name]
        assert [w.H, w.Dk] == facts["g_shape_tail"]["value"]


def test_generator_is_seeded_and_shaped():
    a = synth.make_chunk_inputs(1, 100, 3, 16, 8, seed=5, dtype="bf16", init_state=True)
    b = synth.make_chunk_inputs(1, 100, 3, 16, 8, seed=5, dtype="bf16", init_state=True)
    for key in ("q", "k", "v", "g", "beta", "initial_state"):
        assert torch.equal(a[key], b[key])
    assert a["q"].shape == (1, 100, 3, 16) and a["v"].shape == (1, 100, 3, 8)
    assert a["g"].shape == (1, 100, 3, 16) and a["beta"].shape == (1, 100, 3)
    assert a["q"].dtype == torch.bfloat16 and a["initial_state"].dtype == torch.float32
    g = a["g"].float()
    assert float(g.max()) <= 0.0 and float(g.min()) >= synth.GATE_LOWER_BOUND
    beta = a["beta"].float()
    assert float(beta.min()) > 0.0 and float(beta.max()) < 1.0
    kn = torch.linalg.vector_norm(a["k"].float(), dim=-1)
    assert torch.allclose(kn, torch.ones_like(kn), atol=2e-2)    # unit norm before the bf16 cast
    assert abs(float(a["initial_state"].std()) - 0.02) < 2e-3


def test_packed_lengths_cover_the_stated_range():
    rng = np.random.default_rng(0)
    lens = synth.packed_lengths(rng, 20000, 128, 8192)
    assert lens.min() == 128 and lens.max() == 8192
    d = synth.make_chunk_inputs(1, 0, 2, 16, 16, seed=3, n_seqs=16, len_lo=128, len_hi=8192,
                                dtype="f32")
    cu = d["cu_seqlens"].numpy()
    assert cu.dtype == np.int32 and cu[0] == 0 and np.all(np.diff(cu) >= 128)
    assert d["q"].shape[1] == cu[-1]


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)], dtype=np.float32)
    t = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(t, [1.0, 1.0 + 2.0 ** -6, -1.0])
