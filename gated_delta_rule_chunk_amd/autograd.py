"""torch.autograd entry points over the C ABI, for training with loss.backward().

Each pairs one of the library's forward calls with its backward call:
``chunk_kda`` (kda_chunk_fwd / kda_chunk_bwd), ``chunk_kda_prologue``
(kda_chunk_fwd_prologue / kda_chunk_bwd_prologue) and ``chunk_kda_conv``
(kda_chunk_fwd_conv / kda_chunk_bwd_conv). The name follows the compute path
the ISEEKYAN/k3 README names for the KDA layer (its compute-path paragraph);
the arguments are this library's. With ``segments`` > 1 the forward runs the
intra-sequence split (kda_chunk_fwd_split, _split_prologue), which computes the
same function, so its gradient is the same backward call's. Every step runs in
the library's kernels: this module saves the inputs, routes the incoming
gradients to the backward call and casts the float32 gradients to each input's
dtype.
"""
import torch

from . import (chunk_bwd, chunk_bwd_conv, chunk_bwd_prologue, chunk_fwd, chunk_fwd_conv, chunk_fwd_prologue,
               chunk_fwd_split, chunk_fwd_split_prologue)


def _contig(t):
    return None if t is None else t.contiguous()


def _cast(grad, like):
    return None if grad is None or like is None else grad.to(like.dtype)


class _Chunk(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, g, beta, initial_state, cu_seqlens, scale, chunk_size, segments):
        if segments > 1:
            o, fin = chunk_fwd_split(q, k, v, g, beta, segments, initial_state=initial_state, cu_seqlens=cu_seqlens,
                                     chunk_size=chunk_size, scale=scale)
        else:
            o, fin = chunk_fwd(q, k, v, g, beta, initial_state=initial_state, cu_seqlens=cu_seqlens,
                               chunk_size=chunk_size, scale=scale)
        ctx.save_for_backward(q, k, v, g, beta, initial_state, cu_seqlens)
        ctx.scale = scale
        return o, fin

    @staticmethod
    def backward(ctx, d_o, d_fin):
        q, k, v, g, beta, s0, cu = ctx.saved_tensors
        dq, dk, dv, dg, db, d0 = chunk_bwd(q, k, v, g, beta, _contig(d_o), initial_state=s0,
                                           d_final_state=_contig(d_fin), cu_seqlens=cu, scale=ctx.scale,
                                           want_d_initial=s0 is not None)
        return (_cast(dq, q), _cast(dk, k), _cast(dv, v), _cast(dg, g), _cast(db, beta), d0, None, None, None, None)


class _ChunkPrologue(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q_raw, k_raw, v, g_logit, beta_logit, A_log, dt_bias, initial_state, cu_seqlens, scale, lb,
                eps, chunk_size, segments):
        if segments > 1:
            o, fin = chunk_fwd_split_prologue(q_raw, k_raw, v, g_logit, beta_logit, A_log, dt_bias, segments,
                                              gate_lower_bound=lb, l2_eps=eps, initial_state=initial_state,
                                              cu_seqlens=cu_seqlens, chunk_size=chunk_size, scale=scale)
        else:
            o, fin = chunk_fwd_prologue(q_raw, k_raw, v, g_logit, beta_logit, A_log, dt_bias, gate_lower_bound=lb,
                                        l2_eps=eps, initial_state=initial_state, cu_seqlens=cu_seqlens,
                                        chunk_size=chunk_size, scale=scale)
        ctx.save_for_backward(q_raw, k_raw, v, g_logit, beta_logit, A_log, dt_bias, initial_state, cu_seqlens)
        ctx.args = (scale, lb, eps)
        return o, fin

    @staticmethod
    def backward(ctx, d_o, d_fin):
        q, k, v, gl, bl, A_log, dt_bias, s0, cu = ctx.saved_tensors
        scale, lb, eps = ctx.args
        dq, dk, dv, dg, db, dA, dbias, d0 = chunk_bwd_prologue(
            q, k, v, gl, bl, A_log, dt_bias, _contig(d_o), gate_lower_bound=lb, l2_eps=eps, initial_state=s0,
            d_final_state=_contig(d_fin), cu_seqlens=cu, scale=scale, want_d_initial=s0 is not None)
        return (_cast(dq, q), _cast(dk, k), _cast(dv, v), _cast(dg, gl), _cast(db, bl), dA, dbias, d0,
                None, None, None, None, None, None)


class _ChunkConv(torch.autograd.Function):
    @staticmethod
    def forward(ctx, xq, xk, xv, wq, wk, wv, g_logit, beta_logit, A_log, dt_bias, initial_state, cs_q, cs_k, cs_v,
                cu_seqlens, scale, lb, eps, activation, chunk_size):
        o, fin, conv_fin = chunk_fwd_conv(xq, xk, xv, wq, wk, wv, g_logit, beta_logit, A_log, dt_bias,
                                          conv_states=(cs_q, cs_k, cs_v), activation=activation,
                                          gate_lower_bound=lb, l2_eps=eps, initial_state=initial_state,
                                          cu_seqlens=cu_seqlens, chunk_size=chunk_size, scale=scale)
        ctx.save_for_backward(xq, xk, xv, wq, wk, wv, g_logit, beta_logit, A_log, dt_bias, initial_state, cs_q,
                              cs_k, cs_v, cu_seqlens)
        ctx.args = (scale, lb, eps, activation)
        return (o, fin) + tuple(conv_fin)

    @staticmethod
    def backward(ctx, d_o, d_fin, d_cq, d_ck, d_cv):
        xq, xk, xv, wq, wk, wv, gl, bl, A_log, dt_bias, s0, cs_q, cs_k, cs_v, cu = ctx.saved_tensors
        scale, lb, eps, act = ctx.args
        gr = chunk_bwd_conv(xq, xk, xv, wq, wk, wv, gl, bl, A_log, dt_bias, _contig(d_o),
                            conv_states=(cs_q, cs_k, cs_v), d_conv_final=tuple(_contig(t) for t in (d_cq, d_ck, d_cv)),
                            activation=act, gate_lower_bound=lb, l2_eps=eps, initial_state=s0,
                            d_final_state=_contig(d_fin), cu_seqlens=cu, scale=scale, want_d_initial=s0 is not None)
        return (_cast(gr["xq"], xq), _cast(gr["xk"], xk), _cast(gr["xv"], xv), gr["wq"], gr["wk"], gr["wv"],
                _cast(gr["g_logit"], gl), _cast(gr["beta_logit"], bl), gr["A_log"], gr["dt_bias"], gr["initial_state"],
                gr["conv_state_q"] if cs_q is not None else None, gr["conv_state_k"] if cs_k is not None else None,
                gr["conv_state_v"] if cs_v is not None else None, None, None, None, None, None, None)


def chunk_kda(q, k, v, g, beta, initial_state=None, cu_seqlens=None, scale=1.0, chunk_size=0, segments=1):
    """Differentiable ``chunk_fwd`` (``chunk_fwd_split`` with ``segments`` >
    1): returns (o, final_state). Gradients reach q, k, v, g, beta and
    initial_state (kda_chunk_bwd)."""
    return _Chunk.apply(q, k, v, g, beta, initial_state, cu_seqlens, float(scale), int(chunk_size), int(segments))


def chunk_kda_prologue(q_raw, k_raw, v, g_logit, beta_logit, A_log, dt_bias, initial_state=None, cu_seqlens=None,
                       scale=1.0, gate_lower_bound=-5.0, l2_eps=1e-6, chunk_size=0, segments=1):
    """Differentiable ``chunk_fwd_prologue`` (``chunk_fwd_split_prologue``
    with ``segments`` > 1): returns (o, final_state). Gradients reach the raw
    projections, v, A_log, dt_bias and initial_state (kda_chunk_bwd_prologue)."""
    return _ChunkPrologue.apply(q_raw, k_raw, v, g_logit, beta_logit, A_log, dt_bias, initial_state, cu_seqlens,
                                float(scale), float(gate_lower_bound), float(l2_eps), int(chunk_size), int(segments))


def chunk_kda_conv(xq, xk, xv, wq, wk, wv, g_logit, beta_logit, A_log, dt_bias, conv_states=None, initial_state=None,
                   cu_seqlens=None, scale=1.0, activation=True, gate_lower_bound=-5.0, l2_eps=1e-6, chunk_size=0):
    """Differentiable ``chunk_fwd_conv``: returns (o, final_state, (conv_q,
    conv_k, conv_v) final conv states). Gradients reach the pre-convolution
    projections, the taps, the conv states, the gate logits and parameters and
    initial_state (kda_chunk_bwd_conv)."""
    cs = (None, None, None) if conv_states is None else tuple(conv_states)
    o, fin, cq, ck, cv = _ChunkConv.apply(xq, xk, xv, wq, wk, wv, g_logit, beta_logit, A_log, dt_bias, initial_state,
                                          cs[0], cs[1], cs[2], cu_seqlens, float(scale), float(gate_lower_bound),
                                          float(l2_eps), bool(activation), int(chunk_size))
    return o, fin, (cq, ck, cv)
