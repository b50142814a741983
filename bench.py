"""Benchmark: KDA chunked forward on the K3 layer shape, one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-decode] [--no-backward] [--no-split]
                    [--only split|backward|conv|decode|f32]

One step = one kda_chunk_fwd call over a K3-shaped batch: B=1, T=4096, H=96,
d_k=d_v=128, bf16 inputs, zero initial state, output plus final state. The
workload is specified with 64-row chunks; the bf16 kernel always works in
16-row chunks (the chunk size changes only the rounding, never the result of
the recurrence), so the call passes chunk_size=0 (the kernel's own). Inputs are seeded synthetic tensors (synth.WORKLOADS["k3_t4096"]),
resident in HBM before timing; two input sets alternate so the 256 MB
Infinity Cache cannot serve a step from the previous one. Before the W
warm-up steps the call runs back to back for a fixed 0.25 s (untimed) so that
the GPU reaches its loaded clocks; an idle MI355X needs about a hundred
launches for that, and the first launches run up to 20% slower.

Prints one JSON line. ``value`` is tokens/s of the forward (T / seconds per
step). ``roofline`` is for the chunk kernel: algorithmic HBM bytes per launch
(q,k,v,g,o at 256 B per token-head each, beta at 2 B, the fp32 final state)
over its average launch time, measured with HIP events on the launch stream.
``f32`` times the same forward with float32 inputs and output (the float32
chunk kernel, 16-row chunks, products as f32 MFMA) against the fp32 matrix peak.
``prologue`` times the same forward from raw projections with the gate, beta
and L2-normalisation prologue fused into the chunk kernel
(kda_chunk_fwd_prologue). ``short_conv`` times the kernel-4 convolution of the
q, k and v projections (kda_short_conv), the chain convolution ->
prologue forward, and the same chain as one call (kda_chunk_fwd_conv, ``fused``). ``mfma`` gives the same launches against the bf16 dense matrix-core peak with
the algorithmic flop count of the chunk form at C=64 counted over full tiles,
a fixed count that does not depend on the chunk size the kernel uses. ``backward`` times kda_chunk_bwd on
the same workload with output and final-state cotangents, against the fp32
matrix-core peak (its products run as float32 MFMA) with the algorithmic flop
count of the chunked backward (recompute included), plus the fp64 oracle's
backward on the same workload; its ``from_raw_projections`` entry times the
backward through the gate, beta and L2-norm prologue (kda_chunk_bwd_prologue), and its ``from_conv`` entry
the backward from the pre-convolution projections (kda_chunk_bwd_conv). ``split`` times the intra-sequence split
(kda_chunk_fwd_split, 10 segments) on 12 heads at T=32768 against the unsplit
call. ``decode`` times kda_recurrent_step on
256 rows x 96 heads against an fp32 state cache (HBM-bound); its
``from_conv`` entry times one token from the projections before the short
convolution (kda_recurrent_step_conv: convolution step, prologue and state
update in one kernel) beside the same work as four calls. ``cpu_baseline``
times the fp64 CPU oracle (C, OpenMP over heads) on the same forward workload,
repeated until about ten seconds of wall time have passed.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gated_delta_rule_chunk_amd as kda  # noqa: E402
import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
F32_PEAK_TFLOPS = 157.3        # MI355X fp32, dense MFMA and vector ALU alike, TFLOP/s
METRIC = "KDA fwd tokens/s at H=96,d=128 (bf16); MFMA util % and decode HBM GB/s"
CHUNK_KERNEL_SRC = os.path.join(ROOT, "gated_delta_rule_chunk_amd", "csrc", "chunk_mfma.hip")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "chunk_mfma_k3_t4096_traffic.md")
BWD_KERNEL_SRC = os.path.join(ROOT, "gated_delta_rule_chunk_amd", "csrc", "chunk_bwd.hip")
BWD_SUMMARY = os.path.join(ROOT, "profiles", "chunk_bwd_k3_t4096.md")


def fwd_bytes(T, H, Dk, Dv, n_states_out, n_states_in=0, elem=2):
    per_tok_head = elem * (3 * Dk + 2 * Dv) + elem          # q,k,g,v in, o out, beta
    return T * H * per_tok_head + 4 * Dk * Dv * H * (n_states_out + n_states_in)


def fwd_flops(T, H, Dk, Dv, C=64):
    """Full-tile flop count of the chunk form at chunk C, per launch."""
    return T * H * (2 * C * (3 * Dk + 2 * Dv) + 6 * Dk * Dv)


def kernel_source_hash():
    return hashlib.sha256(open(CHUNK_KERNEL_SRC, "rb").read()).hexdigest()[:16]


def bwd_source_hash():
    return hashlib.sha256(open(BWD_KERNEL_SRC, "rb").read()).hexdigest()[:16]


def read_bwd_traffic():
    """HBM bytes per backward call from the committed counter summary, if it was
    taken on the current backward source; otherwise None."""
    if not os.path.exists(BWD_SUMMARY):
        return None
    text = open(BWD_SUMMARY).read()
    m_hash = re.search(r"bwd_source_sha256:\s*([0-9a-f]+)", text)
    m_val = re.search(r"(?m)^bwd_traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_val or m_hash.group(1) != bwd_source_hash():
        return None
    return float(m_val.group(1))


def read_traffic(key="traffic_bytes_per_launch"):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; otherwise None. ``key`` selects the
    plain kernel's or the prologue kernel's figure."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    text = open(TRAFFIC_SUMMARY).read()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    m_val = re.search(r"(?m)^" + key + r":\s*([0-9.eE+]+)", text)
    if not m_hash or not m_val or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_val.group(1))


CSRC = os.path.join(ROOT, "gated_delta_rule_chunk_amd", "csrc")
# per-leg counter summaries: (file, the kernel sources the figure depends on)
LEG_TRAFFIC = {
    "decode": ("recurrent_step_k3_decode_b256_traffic.md", ("recurrent_step.hip",)),
    "short_conv": ("short_conv_k3_t4096_traffic.md", ("short_conv.hip",)),
    "split": ("chunk_fwd_split_h12_t32768_traffic.md", ("split.hip", "chunk_mfma.hip")),
    "f32": ("chunk_generic_k3_t4096_f32.md", ("chunk_generic.hip",)),
}


def leg_source_hash(leg):
    h = hashlib.sha256()
    for name in LEG_TRAFFIC[leg][1]:
        h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()[:16]


def read_leg_traffic(leg, key="traffic_bytes_per_step"):
    """HBM bytes per step of a secondary leg (decode, short_conv, split, f32) from its
    committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary, if it was taken on the
    current sources of its kernels; otherwise None."""
    path = os.path.join(ROOT, "profiles", LEG_TRAFFIC[leg][0])
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"sources_sha256:\s*([0-9a-f]+)", text)
    m_val = re.search(r"(?m)^" + key + r":\s*([0-9.eE+]+)", text)
    if not m_hash or not m_val or m_hash.group(1) != leg_source_hash(leg):
        return None
    return float(m_val.group(1))


MFMA_SUMMARY = os.path.join(ROOT, "profiles", "chunk_mfma_k3_t4096_mfma_counters.md")


def read_mfma_counters():
    """The counter-measured matrix-core figures of the chunk kernel (rocprofv3's
    MfmaUtil and MfmaFlopsBF16, per launch) from the committed summary, if it
    was taken on the current kernel source; otherwise None."""
    if not os.path.exists(MFMA_SUMMARY):
        return None
    text = open(MFMA_SUMMARY).read()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    m_util = re.search(r"(?m)^mfma_util_pct:\s*([0-9.eE+]+)", text)
    m_fl = re.search(r"(?m)^mfma_flops_bf16_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_hash and m_util and m_fl) or m_hash.group(1) != kernel_source_hash():
        return None
    return {"mfma_busy_pct": float(m_util.group(1)), "mfma_flops_bf16_per_launch": float(m_fl.group(1)),
            "what": "rocprofv3 MfmaUtil (matrix-core busy cycles over all SIMDs of the chip) and MfmaFlopsBF16 "
                    "(executed bf16 MFMA flops, identity and zero-padded tiles included)"}


SETTLE_S = 0.25


def settle_clocks(fn, seconds=SETTLE_S):
    """Run the call back to back for `seconds` of wall time, untimed. An idle
    MI355X runs at low clocks and needs about a hundred back-to-back launches
    of this kernel (~25 ms) to reach its loaded clocks; launches timed before
    that measure the ramp, not the kernel."""
    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            fn(i)
            i += 1
        torch.cuda.synchronize()
    return i


def time_launches(fn, steps, warmup, stream):
    """Clock settling (settle_clocks), W warm-up calls, then exactly `steps`
    timed calls back to back, bracketed by device synchronisation. One HIP
    event on the launch stream before the first call and one after every
    call: the K intervals between consecutive events are the per-call
    durations, their mean is the average launch duration over the timed region
    and their median the median call. Returns (wall seconds, per-call ms list,
    average ms)."""
    settle_clocks(fn)
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        fn(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]      # ms
    avg_ms = ev[0].elapsed_time(ev[steps]) / steps
    return wall, per, avg_ms


def bench_forward(steps, warmup):
    w = synth.WORKLOADS["k3_t4096"]
    dev = torch.device("cuda:0")
    sets = []
    for s in range(2):
        inp = synth.make_chunk_inputs(w.B, w.T, w.H, w.Dk, w.Dv, seed=w.seed + 1000 * s, dtype=w.dtype)
        sets.append({k: (None if v is None else v.to(dev)) for k, v in inp.items()})
    o = torch.empty((w.B, w.T, w.H, w.Dv), dtype=torch.bfloat16, device=dev)
    fin = torch.empty((w.B, w.H, w.Dk, w.Dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        d = sets[i % 2]
        kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk_size=0, out=o,
                      final_state=fin)

    wall, per, batch = time_launches(step, steps, warmup, stream)
    if not (torch.isfinite(o.float()).all() and torch.isfinite(fin).all()):
        raise RuntimeError("non-finite forward output")
    return w, wall, per, batch


def bench_prologue(steps, warmup):
    """The same forward from raw projections with the gate, beta and L2-norm
    prologue fused into the chunk kernel (kda_chunk_fwd_prologue)."""
    w = synth.WORKLOADS["k3_t4096"]
    dev = torch.device("cuda:0")
    sets = []
    for s in range(2):
        inp = synth.make_prologue_inputs(w.B, w.T, w.H, w.Dk, w.Dv, seed=w.seed + 1000 * s, dtype=w.dtype)
        sets.append({k: (None if v is None else v.to(dev)) for k, v in inp.items()})
    o = torch.empty((w.B, w.T, w.H, w.Dv), dtype=torch.bfloat16, device=dev)
    fin = torch.empty((w.B, w.H, w.Dk, w.Dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        d = sets[i % 2]
        kda.chunk_fwd_prologue(d["q_raw"], d["k_raw"], d["v"], d["g_logit"], d["beta_logit"], d["A_log"],
                               d["dt_bias"], gate_lower_bound=synth.GATE_LOWER_BOUND, l2_eps=1e-6,
                               out=o, final_state=fin)

    wall, per, batch = time_launches(step, steps, warmup, stream)
    if not (torch.isfinite(o.float()).all() and torch.isfinite(fin).all()):
        raise RuntimeError("non-finite prologue forward output")
    kern_ms = float(batch)
    # the raw projections have the inputs' sizes; A_log and dt_bias add 4 B per channel
    nbytes = fwd_bytes(w.T, w.H, w.Dk, w.Dv, n_states_out=1) + 4 * w.Dk * (1 + w.H)
    gbs = nbytes / (kern_ms * 1e-3) / 1e9
    return {"workload": "k3_t4096 from raw projections: q, k unnormalised, gate and beta logits, "
                        "A_log [128], dt_bias [96*128]; gate lb*sigmoid(exp(A_log)*(logit+dt_bias)), lb=-5, "
                        "L2 eps 1e-6",
            "ms_per_step": wall / steps * 1e3, "tokens_per_s": w.T / (wall / steps), "kernel_ms": kern_ms,
            "kernel_ms_median": float(np.median(per)),
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": read_traffic("prologue_traffic_bytes_per_launch")},
            "algorithmic_bytes_per_launch": nbytes}


def bench_f32(steps, warmup):
    """The same forward with float32 inputs (q, k, v, g, beta, o all fp32):
    the float32 chunk kernel at its default 16-row chunks, whose dense
    products run as f32 MFMA. The roofline is the fp32 matrix peak with the
    full-tile flop count of the chunk form at C=16; the HBM rate of the same
    launches is given beside it."""
    w = synth.WORKLOADS["k3_t4096"]
    dev = torch.device("cuda:0")
    sets = []
    for s in range(2):
        inp = synth.make_chunk_inputs(w.B, w.T, w.H, w.Dk, w.Dv, seed=w.seed + 1000 * s, dtype="f32")
        sets.append({k: (None if v is None else v.to(dev)) for k, v in inp.items()})
    o = torch.empty((w.B, w.T, w.H, w.Dv), dtype=torch.float32, device=dev)
    fin = torch.empty((w.B, w.H, w.Dk, w.Dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        d = sets[i % 2]
        kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], chunk_size=0, out=o, final_state=fin)

    wall, per, batch = time_launches(step, steps, warmup, stream)
    if not (torch.isfinite(o).all() and torch.isfinite(fin).all()):
        raise RuntimeError("non-finite float32 forward output")
    kern_ms = float(batch)
    nflops = fwd_flops(w.T, w.H, w.Dk, w.Dv, C=16)
    nbytes = fwd_bytes(w.T, w.H, w.Dk, w.Dv, n_states_out=1, elem=4)
    tflops = nflops / (kern_ms * 1e-3) / 1e12
    gbs = nbytes / (kern_ms * 1e-3) / 1e9
    return {"workload": "k3_t4096 with float32 q, k, v, g, beta and o (float32 chunk kernel, 16-row chunks)",
            "ms_per_step": wall / steps * 1e3, "tokens_per_s": w.T / (wall / steps), "kernel_ms": kern_ms,
            "kernel_ms_median": float(np.median(per)),
            "roofline": {"bound": "mfma", "achieved": tflops, "peak": F32_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": tflops / F32_PEAK_TFLOPS, "traffic": read_leg_traffic("f32")},
            "flops_per_launch": nflops, "hbm_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "algorithmic_bytes_per_launch": nbytes}


def bench_conv(steps, warmup):
    """The short causal convolution (kernel 4, SiLU) of the q, k and v
    projections at k3_t4096 (kda_short_conv, three launches per step), and the
    chain convolution -> fused-prologue forward."""
    w = synth.WORKLOADS["k3_t4096"]
    dev = torch.device("cuda:0")
    C = w.H * w.Dk
    sets = []
    for s in range(2):
        inp = synth.make_prologue_inputs(w.B, w.T, w.H, w.Dk, w.Dv, seed=w.seed + 1000 * s, dtype=w.dtype)
        sets.append({k: (None if v is None else v.to(dev)) for k, v in inp.items()})
    rng = np.random.default_rng(w.seed)
    weights = [torch.from_numpy((0.5 * rng.standard_normal((C, 4))).astype(np.float32)).to(dev) for _ in range(3)]
    ys = [torch.empty((w.B, w.T, w.H, w.Dk), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    states = [torch.empty((w.B, 3, C), dtype=torch.float32, device=dev) for _ in range(3)]
    o = torch.empty((w.B, w.T, w.H, w.Dv), dtype=torch.bfloat16, device=dev)
    fin = torch.empty((w.B, w.H, w.Dk, w.Dv), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def conv(i):
        d = sets[i % 2]
        for j, name in enumerate(("q_raw", "k_raw", "v")):
            kda.short_conv(d[name], weights[j], activation=True, out=ys[j], final_state=states[j])

    def chain(i):
        conv(i)
        d = sets[i % 2]
        kda.chunk_fwd_prologue(ys[0], ys[1], ys[2], d["g_logit"], d["beta_logit"], d["A_log"], d["dt_bias"],
                               gate_lower_bound=synth.GATE_LOWER_BOUND, l2_eps=1e-6, out=o, final_state=fin)

    ws_f = torch.empty((kda.chunk_fwd_conv_workspace_bytes(w.B, w.T, w.H, w.Dk, w.Dv, torch.bfloat16,
                                                           synth.GATE_LOWER_BOUND),), dtype=torch.uint8, device=dev)

    def fused(i):
        d = sets[i % 2]
        kda.chunk_fwd_conv(d["q_raw"], d["k_raw"], d["v"], *weights, d["g_logit"], d["beta_logit"], d["A_log"],
                           d["dt_bias"], activation=True, gate_lower_bound=synth.GATE_LOWER_BOUND, l2_eps=1e-6,
                           out=o, final_state=fin, conv_states_out=states, workspace=ws_f)

    # backward of the three convolutions: fp32 cotangents of y, gradients of x, the taps and the initial state
    gen = torch.Generator(device="cpu").manual_seed(w.seed + 11)
    dys = [torch.randn((w.B, w.T, C), generator=gen).to(dev) for _ in range(3)]
    dxs = [torch.empty((w.B, w.T, C), dtype=torch.float32, device=dev) for _ in range(3)]
    ws_b = torch.empty((kda.short_conv_bwd_workspace_bytes(w.B, w.T, C),), dtype=torch.uint8, device=dev)
    grads = {}

    def conv_bwd(i):
        d = sets[i % 2]
        for j, name in enumerate(("q_raw", "k_raw", "v")):
            grads[j] = kda.short_conv_bwd(d[name], weights[j], dys[j], activation=True, workspace=ws_b,
                                          out=dxs[j])

    _, conv_per, conv_ms = time_launches(conv, steps, warmup, stream)
    wall, chain_per, _ = time_launches(chain, steps, warmup, stream)
    if not (torch.isfinite(o.float()).all() and torch.isfinite(fin).all()):
        raise RuntimeError("non-finite conv chain output")
    wall_f, fused_per, _ = time_launches(fused, steps, warmup, stream)
    _, bwd_per, bwd_ms = time_launches(conv_bwd, steps, warmup, stream)
    if not (torch.isfinite(o.float()).all() and torch.isfinite(fin).all()):
        raise RuntimeError("non-finite fused conv forward output")
    if not all(torch.isfinite(t).all() for g in grads.values() for t in g if t is not None):
        raise RuntimeError("non-finite conv backward output")
    # per projection: x (2 B) and dy (4 B) read, dx (4 B) written per token-channel, the taps and their
    # gradient, the initial-state gradient; the per-block tap partials (16 B per channel per 64 tokens,
    # written then read) are counted too
    nblk = kda.short_conv_bwd_workspace_bytes(w.B, w.T, C) // (16 * C)
    bwd_bytes = 3 * (w.B * w.T * C * 10 + 2 * C * 4 * 4 + w.B * 3 * C * 4 + 2 * nblk * C * 16)
    bwd_gbs = bwd_bytes / (float(bwd_ms) * 1e-3) / 1e9
    # per projection: x read and y written at 2 B per token-channel, the weights and the final state
    nbytes = 3 * (2 * w.B * w.T * C * 2 + C * 4 * 4 + w.B * 3 * C * 4)
    gbs = nbytes / (float(conv_ms) * 1e-3) / 1e9
    return {"workload": "k3_t4096: causal depthwise conv (kernel 4, SiLU) of q, k, v, each [1,4096,96*128] bf16, "
                        "with the final conv state",
            "ms_per_step": float(conv_ms), "ms_median": float(np.median(conv_per)),
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": read_leg_traffic("short_conv")},
            "algorithmic_bytes_per_step": nbytes,
            "chain": {"steps": "conv of q, k, v then the fused-prologue forward",
                      "ms_per_step": wall / steps * 1e3, "ms_median": float(np.median(chain_per)),
                      "tokens_per_s": w.T / (wall / steps)},
            "fused": {"steps": "kda_chunk_fwd_conv: the same chain in one call (v convolved inside the chunk "
                                "kernel, q and k by the streaming convolution), final conv states included",
                      "ms_per_step": wall_f / steps * 1e3, "ms_median": float(np.median(fused_per)),
                      "tokens_per_s": w.T / (wall_f / steps)},
            "backward": {"steps": "kda_short_conv_bwd of q, k, v (fp32 dy; dx, dweight, d_state)",
                         "ms_per_step": float(bwd_ms), "ms_median": float(np.median(bwd_per)),
                         "roofline": {"bound": "hbm", "achieved": bwd_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": bwd_gbs / HBM_PEAK_GBS,
                                      "traffic": read_leg_traffic("short_conv", "bwd_traffic_bytes_per_step")},
                         "algorithmic_bytes_per_step": bwd_bytes}}


def bench_decode(steps, warmup):
    cfg = synth.DECODE
    Nb, H, Dk, Dv = cfg["Nb"], cfg["H"], cfg["Dk"], cfg["Dv"]
    dev = torch.device("cuda:0")
    cache = synth.make_decode_cache(Nb, H, Dk, Dv, seed=cfg["seed"]).to(dev)
    ins = [{k: v.to(dev) for k, v in synth.make_decode_step(Nb, H, Dk, Dv, cfg["seed"], s).items()}
           for s in range(4)]
    o = torch.empty((Nb, H, Dv), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        d = ins[i % 4]
        kda.recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], cache, out=o)

    wall, per, batch = time_launches(step, steps, warmup, stream)
    if not torch.isfinite(cache).all():
        raise RuntimeError("non-finite decode state")
    step_bytes = 2 * Nb * H * Dk * Dv * 4 + Nb * H * (2 * (3 * Dk + Dv) + 2 + 2 * Dv)
    avg_ms = float(batch)
    gbs = step_bytes / (avg_ms * 1e-3) / 1e9

    # one generated token from the projections before the short convolution: the convolution step of q, k and
    # v over their caches, the gate/beta/normalisation prologue and the state update in one kernel, against the
    # same work as three convolution steps and the prologue step
    raw = [{k: v.to(dev) for k, v in synth.make_decode_raw_step(Nb, H, Dk, Dv, cfg["seed"], s).items()}
           for s in range(4)]
    A_log, dt_bias = (t.to(dev) for t in synth.make_gate_params(H, Dk, cfg["seed"]))
    Cs = (H * Dk, H * Dk, H * Dv)
    taps = [synth.make_conv_taps(C, cfg["seed"], j).to(dev) for j, C in enumerate(Cs)]
    conv = [synth.make_conv_cache(Nb, C, cfg["seed"], j).to(dev) for j, C in enumerate(Cs)]
    ys = [torch.empty((Nb, H, D), dtype=torch.bfloat16, device=dev) for D in (Dk, Dk, Dv)]

    def fused(i):
        d = raw[i % 4]
        kda.recurrent_step_conv(d["q_raw"], d["k_raw"], d["v"], *taps, conv, d["g_logit"], d["beta_logit"], A_log,
                                dt_bias, cache, activation=True, gate_lower_bound=synth.GATE_LOWER_BOUND,
                                l2_eps=1e-6, out=o)

    def chain(i):
        d = raw[i % 4]
        for j, name in enumerate(("q_raw", "k_raw", "v")):
            kda.short_conv_step(d[name], taps[j], conv[j], activation=True, out=ys[j])
        kda.recurrent_step_prologue(ys[0], ys[1], ys[2], d["g_logit"], d["beta_logit"], A_log, dt_bias, cache,
                                    gate_lower_bound=synth.GATE_LOWER_BOUND, l2_eps=1e-6, out=o)

    _, fper, fms = time_launches(fused, steps, warmup, stream)
    _, cper, cms = time_launches(chain, steps, warmup, stream)
    if not (torch.isfinite(cache).all() and torch.isfinite(o.float()).all()):
        raise RuntimeError("non-finite decode state from the convolution inputs")
    # the state read and written, the convolution caches read and written, the inputs, o, the taps and the gate
    # parameters
    conv_bytes = (2 * Nb * H * Dk * Dv * 4 + 2 * Nb * sum(Cs) * 3 * 4 + Nb * H * (2 * (3 * Dk + Dv) + 2 + 2 * Dv)
                  + sum(Cs) * 16 + (Dk + H * Dk) * 4)
    fgbs = conv_bytes / (float(fms) * 1e-3) / 1e9
    return {"workload": f"{cfg['name']}: batch {Nb}, H={H}, d_k=d_v={Dk}, bf16 q/k/v/g/beta, fp32 state cache",
            "ms_per_step": avg_ms, "ms_median": float(np.median(per)), "tokens_per_s": Nb / (avg_ms * 1e-3),
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": read_leg_traffic("decode")},
            "algorithmic_bytes_per_step": step_bytes,
            "from_conv": {"steps": "kda_recurrent_step_conv: the short-convolution step of q, k, v (SiLU, fp32 "
                                   "caches [256,3,96*128]), the gate/beta/normalisation prologue and the state "
                                   "update in one kernel",
                          "ms_per_step": float(fms), "ms_median": float(np.median(fper)),
                          "tokens_per_s": Nb / (float(fms) * 1e-3),
                          "roofline": {"bound": "hbm", "achieved": fgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                       "frac": fgbs / HBM_PEAK_GBS,
                                       "traffic": read_leg_traffic("decode", "conv_traffic_bytes_per_step")},
                          "algorithmic_bytes_per_step": conv_bytes,
                          "chain": {"steps": "kda_short_conv_step x 3, then kda_recurrent_step_prologue",
                                    "ms_per_step": float(cms), "ms_median": float(np.median(cper))}}}


FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 MFMA, TFLOP/s


def bwd_flops(T, H, Dk, Dv, C=16):
    """Algorithmic flops of the chunked backward per launch, recompute included:
    per 16-row chunk and head, 11 state-sized products (2*C*Dk*Dv each: the
    forward re-run's W and state update, W again, Kh dS, the two state-gradient
    products, dO S^T, dW S^T, U dS^T) and the 16x16 ones (KK, P and the four
    pair-gradient products over d_k; T W twice, P^T dO, T^T dU, dO U^T, dY U^T
    over d_v)."""
    per_chunk = 22 * C * Dk * Dv + 12 * C * C * Dk + 12 * C * C * Dv
    return T * H * per_chunk // C


def bwd_bytes(T, H, Dk, Dv, elem=2):
    """Algorithmic HBM bytes of the backward per launch: q, k, g, v, beta and
    d_o read in the input dtype; dq, dk, dg, dv, dbeta written in float32; the
    final-state cotangent read and the initial-state gradient written."""
    per_tok_head = elem * (3 * Dk + 2 * Dv + 1) + 4 * (3 * Dk + Dv + 1)
    return T * H * per_tok_head + 2 * 4 * H * Dk * Dv


def bench_backward(steps, warmup, cpu=True):
    """kda_chunk_bwd on k3_t4096 with an output cotangent and a final-state
    cotangent (seeded, standard deviations 1 and 0.1); float32 gradients."""
    w = synth.WORKLOADS["k3_t4096"]
    dev = torch.device("cuda:0")
    sets = []
    for s in range(2):
        inp = synth.make_chunk_inputs(w.B, w.T, w.H, w.Dk, w.Dv, seed=w.seed + 1000 * s, dtype=w.dtype)
        d_o, dfin = synth.make_cotangents(inp, seed=w.seed + 1000 * s + 7)
        d = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
        d["d_o"], d["d_final"] = d_o.to(dev), dfin.to(dev)
        sets.append(d)
    ws = torch.empty((kda.chunk_bwd_workspace_bytes(w.B, w.T, w.H, w.Dk, w.Dv, w.B, False),), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)
    scale = w.Dk ** -0.5
    out = {}

    def step(i):
        d = sets[i % 2]
        out["g"] = kda.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["d_o"], d_final_state=d["d_final"],
                                 scale=scale, workspace=ws)

    wall, per, batch = time_launches(step, steps, warmup, stream)
    if not all(torch.isfinite(x).all() for x in out["g"]):
        raise RuntimeError("non-finite backward output")
    kern_ms = float(batch)
    nflops = bwd_flops(w.T, w.H, w.Dk, w.Dv)
    nbytes = bwd_bytes(w.T, w.H, w.Dk, w.Dv)
    tflops = nflops / (kern_ms * 1e-3) / 1e12
    res = {"workload": "k3_t4096 backward: B=1, T=4096, H=96, d_k=d_v=128, bf16 q/k/v/g/beta/d_o, "
                       "fp32 final-state cotangent, fp32 dq/dk/dv/dg/dbeta/d_initial",
           "ms_per_step": wall / steps * 1e3, "tokens_per_s": w.T / (wall / steps), "kernel_ms": kern_ms,
           "kernel_ms_median": float(np.median(per)),
           "roofline": {"bound": "mfma", "achieved": tflops, "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": tflops / FP32_MFMA_PEAK_TFLOPS, "traffic": read_bwd_traffic(),
                        "dtype": "f32 (v_mfma_f32_16x16x4f32)"},
           "flops_per_launch": nflops,
           "hbm": {"algorithmic_bytes_per_launch": nbytes,
                   "achieved_GBs": nbytes / (kern_ms * 1e-3) / 1e9,
                   "workspace_bytes_each_way": w.T // 16 * w.H * w.Dk * w.Dv * 4},
           "timed": "one kda_chunk_bwd call: the per-chunk T/P/KK kernel (which also zeroes the atomically "
                    "summed gradients) and the sequential kernel"}
    res["from_raw_projections"] = bench_backward_prologue(steps, warmup)
    res["from_conv"] = bench_backward_conv(steps, warmup)
    if cpu:
        res["cpu_baseline"] = cpu_backward_baseline()
    return res


def bench_backward_prologue(steps, warmup):
    """kda_chunk_bwd_prologue on k3_t4096: the same backward from raw
    projections, through the gate, beta and L2-norm prologue (gradients of the
    raw inputs, A_log and dt_bias)."""
    w = synth.WORKLOADS["k3_t4096"]
    dev = torch.device("cuda:0")
    sets = []
    for s_ in range(2):
        inp = synth.make_prologue_inputs(w.B, w.T, w.H, w.Dk, w.Dv, seed=w.seed + 1000 * s_, dtype=w.dtype)
        d_o, dfin = synth.make_cotangents({"v": inp["v"], "q": inp["q_raw"], "cu_seqlens": None},
                                          seed=w.seed + 1000 * s_ + 7)
        d = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
        d["d_o"], d["d_final"] = d_o.to(dev), dfin.to(dev)
        sets.append(d)
    ws = torch.empty((kda.chunk_bwd_prologue_workspace_bytes(w.B, w.T, w.H, w.Dk, w.Dv, w.B, False),),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    out = {}

    def step(i):
        d = sets[i % 2]
        out["g"] = kda.chunk_bwd_prologue(d["q_raw"], d["k_raw"], d["v"], d["g_logit"], d["beta_logit"], d["A_log"],
                                          d["dt_bias"], d["d_o"], gate_lower_bound=synth.GATE_LOWER_BOUND,
                                          l2_eps=1e-6, d_final_state=d["d_final"], scale=w.Dk ** -0.5,
                                          workspace=ws)

    wall, _, batch = time_launches(step, steps, warmup, stream)
    if not all(torch.isfinite(x).all() for x in out["g"] if x is not None):
        raise RuntimeError("non-finite backward output")
    return {"workload": "k3_t4096 backward from raw projections (gate lb=-5, L2 eps 1e-6): gradients of q_raw, "
                        "k_raw, v, g_logit, beta_logit, A_log, dt_bias and the initial state",
            "ms_per_step": wall / steps * 1e3, "kernel_ms": float(batch),
            "tokens_per_s": w.T / (float(batch) * 1e-3)}


def bench_backward_conv(steps, warmup):
    """kda_chunk_bwd_conv on k3_t4096: the backward from the projections
    before the short convolution (SiLU, zero initial conv states), with the
    convolutions recomputed, the prologue backward and the convolution
    backward of q, k and v in one call."""
    w = synth.WORKLOADS["k3_t4096"]
    dev = torch.device("cuda:0")
    C = w.H * w.Dk
    taps = [synth.make_conv_taps(C, w.seed, j).to(dev) for j in range(3)]
    sets = []
    for s_ in range(2):
        inp = synth.make_prologue_inputs(w.B, w.T, w.H, w.Dk, w.Dv, seed=w.seed + 1000 * s_, dtype=w.dtype)
        d_o, dfin = synth.make_cotangents({"v": inp["v"], "q": inp["q_raw"], "cu_seqlens": None},
                                          seed=w.seed + 1000 * s_ + 7)
        d = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
        d["d_o"], d["d_final"] = d_o.to(dev), dfin.to(dev)
        sets.append(d)
    ws = torch.empty((kda.chunk_bwd_conv_workspace_bytes(w.B, w.T, w.H, w.Dk, w.Dv, w.B, False, torch.bfloat16),),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    out = {}

    def step(i):
        d = sets[i % 2]
        out["g"] = kda.chunk_bwd_conv(d["q_raw"], d["k_raw"], d["v"], *taps, d["g_logit"], d["beta_logit"],
                                      d["A_log"], d["dt_bias"], d["d_o"], activation=True,
                                      gate_lower_bound=synth.GATE_LOWER_BOUND, l2_eps=1e-6,
                                      d_final_state=d["d_final"], scale=w.Dk ** -0.5, workspace=ws)

    wall, per, batch = time_launches(step, steps, warmup, stream)
    if not all(torch.isfinite(x).all() for x in out["g"].values() if x is not None):
        raise RuntimeError("non-finite backward output")
    return {"workload": "k3_t4096 backward from the pre-convolution projections (kernel-4 conv with SiLU, gate "
                        "lb=-5, L2 eps 1e-6): gradients of xq, xk, xv, the taps, the conv states, g_logit, "
                        "beta_logit, A_log, dt_bias and the initial state",
            "ms_per_step": wall / steps * 1e3, "kernel_ms": float(batch), "kernel_ms_median": float(np.median(per)),
            "tokens_per_s": w.T / (float(batch) * 1e-3)}


def bench_split(steps, warmup, segments=10):
    """The intra-sequence split (kda_chunk_fwd_split) on the shape it is for:
    12 heads (one GPU's share of the 96 under 8-way head sharding) at
    T=32768, bf16, initial state ~ N(0, 0.02); against the unsplit call."""
    B, T, H, D = 1, 32768, 12, 128
    dev = torch.device("cuda:0")
    sets = []
    for s_ in range(2):
        inp = synth.make_chunk_inputs(B, T, H, D, D, seed=2 + 1000 * s_, dtype="bf16", init_state=True)
        sets.append({k: (None if v is None else v.to(dev)) for k, v in inp.items()})
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device=dev)
    fin = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty((kda.chunk_fwd_split_workspace_bytes(B, T, H, D, D, B, torch.bfloat16, segments),),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def plain(i):
        d = sets[i % 2]
        kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=d["initial_state"], out=o,
                      final_state=fin)

    def split(i):
        d = sets[i % 2]
        kda.chunk_fwd_split(d["q"], d["k"], d["v"], d["g"], d["beta"], segments, initial_state=d["initial_state"],
                            out=o, final_state=fin, workspace=ws)

    # the same from raw projections (gate, beta and normalisation prologue in every pass)
    A_log, dt_bias = (t.to(dev) for t in synth.make_gate_params(H, D, 2))

    def split_raw(i):
        d = sets[i % 2]
        kda.chunk_fwd_split_prologue(d["q"], d["k"], d["v"], d["g"], d["beta"], A_log, dt_bias, segments,
                                     gate_lower_bound=synth.GATE_LOWER_BOUND, l2_eps=1e-6,
                                     initial_state=d["initial_state"], out=o, final_state=fin, workspace=ws)

    _, _, plain_ms = time_launches(plain, steps, warmup, stream)
    _, raw_per, raw_ms = time_launches(split_raw, steps, warmup, stream)
    if not (torch.isfinite(o.float()).all() and torch.isfinite(fin).all()):
        raise RuntimeError("non-finite split output from raw projections")
    wall, split_per, split_ms = time_launches(split, steps, warmup, stream)
    if not (torch.isfinite(o.float()).all() and torch.isfinite(fin).all()):
        raise RuntimeError("non-finite split output")
    nbytes = fwd_bytes(T, H, D, D, n_states_out=1, n_states_in=1)
    gbs = nbytes / (float(split_ms) * 1e-3) / 1e9
    return {"workload": f"B=1, T={T}, H={H} (12 of the 96 heads), d_k=d_v=128, bf16, initial state N(0,0.02), "
                        f"final state; {segments} segments per sequence",
            "segments": segments, "ms_per_step": float(split_ms), "ms_median": float(np.median(split_per)),
            "tokens_per_s": T / (float(split_ms) * 1e-3),
            "unsplit_ms_per_step": float(plain_ms), "speedup_vs_unsplit": float(plain_ms) / float(split_ms),
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": read_leg_traffic("split")},
            "algorithmic_bytes_per_step": nbytes,
            "timed": "one kda_chunk_fwd_split call: the A and B passes over the segments (one launch), the "
                     "entry-state scan, the correction of the outputs of segments after the first",
            "from_raw_projections": {"steps": "kda_chunk_fwd_split_prologue on the same tensors read as raw "
                                              "projections (q, k unnormalised, gate and beta logits)",
                                     "ms_per_step": float(raw_ms), "ms_median": float(np.median(raw_per))}}


def cpu_backward_baseline(heads=96):
    """The fp64 C oracle's backward on k3_t4096: all 4096 tokens of the first
    `heads` heads (all 96 by default, a few seconds on 16 threads), scaled to
    the whole workload."""
    from oracle import kda_ref
    w = synth.WORKLOADS["k3_t4096"]
    cores = len(os.sched_getaffinity(0))
    omp = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    if omp > 0:
        cores = min(cores, omp)
    inp = synth.make_chunk_inputs(w.B, w.T, w.H, w.Dk, w.Dv, seed=w.seed, dtype=w.dtype)
    d_o, dfin = synth.make_cotangents(inp, seed=w.seed + 7)
    f = {k: inp[k].float().numpy()[:, :, :heads] for k in ("q", "k", "v", "g", "beta")}
    t0 = time.perf_counter()
    kda_ref.c_backward(f["q"], f["k"], f["v"], f["g"], f["beta"], d_o.float().numpy()[:, :, :heads],
                       d_final=dfin.numpy()[:, :heads], scale=w.Dk ** -0.5, nthreads=cores)
    wall = time.perf_counter() - t0
    return {"value": w.T * heads / w.H / wall, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"k3_t4096 backward, all {w.T} tokens of {heads} of the {w.H} heads (fp64 C oracle, "
                      f"OpenMP over heads on {cores} threads), {wall:.1f} s wall, scaled by {heads}/{w.H}"}


def cpu_baseline(min_wall_s=10.0, max_runs=200):
    """The fp64 C oracle over the whole k3_t4096 workload (all heads, all
    tokens), run repeatedly until min_wall_s of wall time has passed."""
    from oracle import kda_ref
    w = synth.WORKLOADS["k3_t4096"]
    cores = len(os.sched_getaffinity(0))
    omp = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    if omp > 0:
        cores = min(cores, omp)
    inp = synth.make_chunk_inputs(w.B, w.T, w.H, w.Dk, w.Dv, seed=w.seed, dtype=w.dtype)
    f = {k: inp[k].float().numpy() for k in ("q", "k", "v", "g", "beta")}
    runs, t0 = 0, time.perf_counter()
    while True:
        kda_ref.c_forward(f["q"], f["k"], f["v"], f["g"], f["beta"], nthreads=cores, want_final=True)
        runs += 1
        wall = time.perf_counter() - t0
        if wall >= min_wall_s or runs >= max_runs:
            break
    t1 = time.perf_counter()
    kda_ref.c_forward(f["q"], f["k"], f["v"], f["g"], f["beta"], nthreads=1, want_final=True)
    single = w.B * w.T / (time.perf_counter() - t1)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": runs * w.B * w.T / wall, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"k3_t4096 whole workload (B=1, T={w.T}, H={w.H}, d=128; all heads and tokens), "
                      f"fp64 C oracle with OpenMP over the {w.H} heads on {cores} threads, {runs} runs "
                      f"in {wall:.1f} s wall",
            "single_thread_value": single, "cpu_model": model}


def copy_calibration(nbytes=1 << 30):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    dev = torch.device("cuda:0")
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).uniform_()
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_each_way": nbytes, "launches": 3}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-split", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--only", choices=["split", "backward", "conv", "decode", "f32"], default=None,
                    help="run one secondary leg alone and print its JSON object (for per-kernel profiles)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    kda.load_library()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.only:
        legs = {"split": lambda: bench_split(args.steps, args.warmup),
                "backward": lambda: bench_backward(args.steps, args.warmup, cpu=False),
                "conv": lambda: bench_conv(args.steps, args.warmup),
                "decode": lambda: bench_decode(args.steps, args.warmup),
                "f32": lambda: bench_f32(args.steps, args.warmup)}
        leg = legs[args.only]()
        print(json.dumps({"only": args.only, **leg}), flush=True)
        return

    w, wall, per, batch = bench_forward(args.steps, args.warmup)
    ms_per_step = wall / args.steps * 1e3
    kern_ms = float(batch)                   # average launch duration over the timed region
    kern_ms_median = float(np.median(per))   # median of the timed calls
    nbytes = fwd_bytes(w.T, w.H, w.Dk, w.Dv, n_states_out=1)
    nflops = fwd_flops(w.T, w.H, w.Dk, w.Dv)
    gbs = nbytes / (kern_ms * 1e-3) / 1e9
    tflops = nflops / (kern_ms * 1e-3) / 1e12
    traffic = read_traffic()
    line = {
        "metric": METRIC,
        "value": w.T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle_s": SETTLE_S,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "k3_t4096: KDA chunked forward, B=1, T=4096, H=96, d_k=d_v=128, "
                               "bf16 q/k/v/g/beta, zero initial state, fp32 final state",
                   "B": w.B, "T": w.T, "H": w.H, "d_k": w.Dk, "d_v": w.Dv,
                   "chunk": 16, "chunk_note": f"specified at C={w.chunk}; the bf16 kernel runs 16-row chunks "
                                             "(changes rounding only)"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": traffic},
        "kernel_ms": kern_ms,
        "kernel_ms_median": kern_ms_median,
        "kernel_ms_min_max": [float(np.min(per)), float(np.max(per))],
        "tokens_per_s_at_median": w.T / (kern_ms_median * 1e-3),
        "algorithmic_bytes_per_launch": nbytes,
        "mfma": {"achieved": tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": tflops / BF16_PEAK_TFLOPS, "flops_per_launch": nflops,
                 "count": "algorithmic, fixed: full 64x64 tiles of the chunk form at C=64, "
                          "T*H*(2*64*(3*d_k+2*d_v)+6*d_k*d_v), whatever chunk the kernel uses",
                 "counter_measured": read_mfma_counters()},
        "published_baseline": "none: the source pages report no KDA throughput on any hardware",
    }
    line["prologue"] = bench_prologue(args.steps, args.warmup)
    line["short_conv"] = bench_conv(args.steps, args.warmup)
    line["f32"] = bench_f32(args.steps, args.warmup)
    if not args.no_split:
        line["split"] = bench_split(args.steps, args.warmup)
    if not args.no_backward:
        line["backward"] = bench_backward(args.steps, args.warmup, cpu=not args.no_cpu_baseline)
    if not args.no_decode:
        line["decode"] = bench_decode(args.steps, args.warmup)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
