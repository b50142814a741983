"""Seeded synthetic KDA inputs (no recurrence arithmetic lives here)."""
from .inputs import (DECODE, GATE_LOWER_BOUND, K3_HEAD_DIM, K3_HEADS, WORKLOADS,  # noqa: F401
                     Workload, as_f32_numpy, make_chunk_inputs, make_cotangents, make_decode_cache, make_prologue_inputs,
                     make_decode_step, make_workload, packed_lengths, make_decode_raw_step, make_gate_params,
                     make_conv_taps, make_conv_cache)
