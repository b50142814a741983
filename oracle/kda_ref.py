"""Plain fp64 CPU oracle for Kimi Delta Attention (KDA).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg of
the benchmark are the only callers. The product path never imports this module
and this module imports nothing from the product package.

KDA is the gated delta rule with a per-channel diagonal decay. For one sequence
and one head, with state S of shape [d_k, d_v], token t does:

    S  <- Diag(exp g_t) S                     (decay, one factor per key channel)
    S  <- (I - beta_t k_t k_t^T) S + beta_t k_t v_t^T
    o_t = scale * S^T q_t                      (read after the update)

Sources: the ISEEKYAN/k3 README names KDA as 69 of the 93 K3 layers and its
"bounded torch recurrence" as the CPU correctness path; the hysenlabs article
"kimi-k3-mlx: a faithful MLX port ...", section "The A_log shape mismatch is a
silent-garbage bug the tests assert", fixes the log-decay g as a
(B,T,96,128) tensor, i.e. per token, head and key channel. The pages print no
equation; the update above is the gated delta rule in its plainest reading
(decay, then erase along k_t, then write beta_t k_t v_t^T; the output uses the
post-update state).

Two implementations, written separately:
  * ``recurrence`` / ``decode_step`` below: NumPy, vectorised over heads only,
    one Python-level step per token;
  * ``c_forward`` / ``c_decode_step``: the plain C loops in kda_ref.c (OpenMP
    over independent (sequence, head) units), loaded with ctypes.
The reverse-mode gradient has the same two forms (``recurrence_backward``,
``c_backward``); both are pinned against central finite differences of the
forward, not against each other alone.
The gate, beta and normalisation prologue that turns raw projections into
(q, k, g, beta) has a NumPy form (``prologue``, then ``recurrence``) and a C
form (``c_prologue_forward``); the reading of the gate it implements is in
``prologue``'s docstring. ``prologue_backward`` is its reverse-mode gradient,
pinned by central differences of prologue-then-recurrence.
Both take inputs as float arrays that hold the GPU's bf16 or fp32 values
exactly, and compute in float64.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda_ref.so")


# ----------------------------------------------------------------------------
# NumPy twin
# ----------------------------------------------------------------------------

def _segments(B, T, cu_seqlens):
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    cu = [int(x) for x in np.asarray(cu_seqlens).reshape(-1)]
    if B != 1 or cu[0] != 0 or cu[-1] != T or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must start at 0, be non-decreasing, end at T, with B == 1")
    return [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]


def token_step(S, q_t, k_t, v_t, g_t, beta_t, scale=1.0):
    """One token for a stack of heads. S [H,Dk,Dv] is updated in place; returns o_t [H,Dv]."""
    S *= np.exp(g_t)[:, :, None]                               # Diag(exp g_t) S
    x = np.einsum("hk,hkv->hv", k_t, S)                        # S^T k_t
    S += (beta_t[:, None, None] * k_t[:, :, None]) * (v_t - x)[:, None, :]
    return scale * np.einsum("hk,hkv->hv", q_t, S)             # S_t^T q_t


def recurrence(q, k, v, g, beta, initial_state=None, cu_seqlens=None, scale=1.0):
    """Sequential fp64 forward. Returns (o [B,T,H,Dv], final_state [N,H,Dk,Dv]).

    q,k,g: [B,T,H,Dk]; v: [B,T,H,Dv]; beta: [B,T,H]; initial_state: [N,H,Dk,Dv]
    or None (zeros); cu_seqlens: [N+1] packed offsets (then B must be 1) or None
    (then N = B). Rows outside every sequence stay zero in o.
    """
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    segs = _segments(B, T, cu_seqlens)
    o = np.zeros((B, T, H, Dv))
    final = np.zeros((len(segs), H, Dk, Dv))
    for n, (b, bos, eos) in enumerate(segs):
        if initial_state is None:
            S = np.zeros((H, Dk, Dv))
        else:
            S = np.array(initial_state[n], dtype=np.float64)
        for t in range(bos, eos):
            o[b, t] = token_step(S, q[b, t], k[b, t], v[b, t], g[b, t], beta[b, t], scale)
        final[n] = S
    return o, final


def recurrence_backward(q, k, v, g, beta, d_o, initial_state=None, d_final=None, cu_seqlens=None,
                        scale=1.0):
    """Reverse-mode gradient of ``recurrence`` (float64), for the scalar loss

        L = sum_t <d_o[t], o[t]> + sum_n <d_final[n], S_final[n]>.

    Walks each sequence backward, differentiating the three steps of
    ``token_step`` in reverse (write, erase-read, decay) with dS = dL/dS_t:

        dS  += scale q_t d_o_t^T                  (o_t = scale S_t^T q_t)
        dq_t = scale S_t d_o_t
        du   = dS^T k_t,   dk_t = dS u            (S_t = S' + k_t u^T)
        dbeta_t = du . (v_t - x),   dv_t = beta_t du,   dx = -beta_t du
        dk_t += S' dx,   dS' = dS + k_t dx^T       (x = S'^T k_t)
        dg_t = rowsum(dS' * S'),   dS = Diag(exp g_t) dS'   (S' = Diag(exp g_t) S_{t-1})

    with u = beta_t (v_t - x). States are kept from a forward pass (small
    inputs only). Returns (dq, dk, dv, dg, dbeta, d_initial [N,H,Dk,Dv]); rows
    outside every sequence are zero.
    """
    q, k, v, g, beta, d_o = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta, d_o))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    segs = _segments(B, T, cu_seqlens)
    dq, dk, dg = (np.zeros((B, T, H, Dk)) for _ in range(3))
    dv = np.zeros((B, T, H, Dv))
    dbeta = np.zeros((B, T, H))
    d_init = np.zeros((len(segs), H, Dk, Dv))
    for n, (b, bos, eos) in enumerate(segs):
        S = np.zeros((H, Dk, Dv)) if initial_state is None else np.array(initial_state[n], dtype=np.float64)
        prev = []                                      # S_{t-1} for each t
        for t in range(bos, eos):
            prev.append(S.copy())
            token_step(S, q[b, t], k[b, t], v[b, t], g[b, t], beta[b, t], scale)
        dS = np.zeros((H, Dk, Dv)) if d_final is None else np.array(d_final[n], dtype=np.float64)
        for t in range(eos - 1, bos - 1, -1):
            a = np.exp(g[b, t])[:, :, None]
            Sd = a * prev[t - bos]
            x = np.einsum("hk,hkv->hv", k[b, t], Sd)
            u = beta[b, t][:, None] * (v[b, t] - x)
            St = Sd + k[b, t][:, :, None] * u[:, None, :]
            dS += scale * q[b, t][:, :, None] * d_o[b, t][:, None, :]
            dq[b, t] = scale * np.einsum("hkv,hv->hk", St, d_o[b, t])
            du = np.einsum("hkv,hk->hv", dS, k[b, t])
            dkt = np.einsum("hkv,hv->hk", dS, u)
            dbeta[b, t] = (du * (v[b, t] - x)).sum(-1)
            dv[b, t] = beta[b, t][:, None] * du
            dx = -beta[b, t][:, None] * du
            dk[b, t] = dkt + np.einsum("hkv,hv->hk", Sd, dx)
            dSd = dS + k[b, t][:, :, None] * dx[:, None, :]
            dg[b, t] = (dSd * Sd).sum(-1)
            dS = a * dSd
        d_init[n] = dS
    return dq, dk, dv, dg, dbeta, d_init


def prologue(q_raw, k_raw, g_logit, beta_logit, A_log, dt_bias, gate_lower_bound=-5.0, l2_eps=1e-6):
    """The gate, beta and normalisation prologue (float64), per token and head.

    The pages fix the gate's parameters and bound but not its formula (hysenlabs
    "kimi-k3-mlx", section "The A_log shape mismatch is a silent-garbage bug the
    tests assert": A_log has one entry per key channel, shared by every head,
    dt_bias one per (head, channel); section "Attention is 93 layers ...":
    gate_lower_bound = -5). The reading implemented, as documented with the
    library:

        q = q_raw / sqrt(|q_raw|^2 + eps)          (over d_k), k likewise
        g = lb * sigmoid(exp(A_log) * (g_logit + dt_bias))
        beta = sigmoid(beta_logit)

    q_raw, k_raw, g_logit [..., H, Dk]; beta_logit [..., H]; A_log [Dk];
    dt_bias [H*Dk]. Returns (q, k, g, beta) as float64.
    """
    q_raw, k_raw, g_logit = (np.asarray(a, dtype=np.float64) for a in (q_raw, k_raw, g_logit))
    beta_logit = np.asarray(beta_logit, dtype=np.float64)
    H, Dk = q_raw.shape[-2:]
    A = np.exp(np.asarray(A_log, dtype=np.float64).reshape(Dk))
    bias = np.asarray(dt_bias, dtype=np.float64).reshape(H, Dk)
    q = q_raw / np.sqrt((q_raw * q_raw).sum(-1, keepdims=True) + l2_eps)
    k = k_raw / np.sqrt((k_raw * k_raw).sum(-1, keepdims=True) + l2_eps)
    g = gate_lower_bound / (1.0 + np.exp(-(A * (g_logit + bias))))
    beta = 1.0 / (1.0 + np.exp(-beta_logit))
    return q, k, g, beta


def prologue_backward(q_raw, k_raw, g_logit, beta_logit, A_log, dt_bias, dq, dk, dg, dbeta,
                      gate_lower_bound=-5.0, l2_eps=1e-6):
    """Reverse-mode gradient of ``prologue`` (float64): given the gradients with
    respect to its outputs (q, k, g, beta), those with respect to its inputs.
    Differentiating each line of the prologue:

        q = x / n, n = sqrt(|x|^2 + eps) (per row):  dx = dq / n - x (x . dq) / n^3
        g = lb * s, s = sigmoid(z), z = exp(A_log[c]) (x + dt_bias[h, c]):
            dz = dg lb s (1 - s);  dx = dz exp(A_log[c]);
            d dt_bias[h, c] = sum over tokens of dz exp(A_log[c]);
            d A_log[c] = sum over tokens and heads of dz z
        beta = sigmoid(y):  dy = dbeta beta (1 - beta)

    Shapes as ``prologue``; returns (dq_raw, dk_raw, dg_logit, dbeta_logit,
    dA_log [Dk], ddt_bias [H*Dk]).
    """
    q_raw, k_raw, g_logit, dq, dk, dg = (np.asarray(a, dtype=np.float64)
                                         for a in (q_raw, k_raw, g_logit, dq, dk, dg))
    beta_logit, dbeta = np.asarray(beta_logit, dtype=np.float64), np.asarray(dbeta, dtype=np.float64)
    H, Dk = q_raw.shape[-2:]
    A = np.exp(np.asarray(A_log, dtype=np.float64).reshape(Dk))
    bias = np.asarray(dt_bias, dtype=np.float64).reshape(H, Dk)

    def l2_back(x, dy):
        n = np.sqrt((x * x).sum(-1, keepdims=True) + l2_eps)
        return dy / n - x * (x * dy).sum(-1, keepdims=True) / n ** 3

    z = A * (g_logit + bias)
    sg = 1.0 / (1.0 + np.exp(-z))
    dz = dg * gate_lower_bound * sg * (1.0 - sg)
    lead = tuple(range(dz.ndim - 2))                       # token axes
    sb = 1.0 / (1.0 + np.exp(-beta_logit))
    return (l2_back(q_raw, dq), l2_back(k_raw, dk), dz * A, dbeta * sb * (1.0 - sb),
            (dz * z).sum(axis=lead + (dz.ndim - 2,)), (dz * A).sum(axis=lead).reshape(H * Dk))


def short_conv(x, w, state=None, cu_seqlens=None, activation=False):
    """Short causal depthwise convolution (kernel 4) over time, float64.

    The pages say KDA applies a short convolution with kernel size 4 on the
    query, key and value projections (hysenlabs "kimi-k3-mlx", section
    "Attention is 93 layers split between KDA and a NoPE gated MLA"); they give
    no formula, weights layout or activation. The reading implemented:
    y[t] = sum_i w[:, i] * x[t - 3 + i] per channel, inputs before a sequence's
    start taken from ``state`` ([N, 3, C]: x[-3], x[-2], x[-1]) or zero, then
    y * sigmoid(y) if ``activation``. x [B, T, C]; w [C, 4]. Returns (y, final
    state [N, 3, C]: the last three inputs of each sequence's window).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, T, C = x.shape
    segs = _segments(B, T, cu_seqlens)
    st0 = None if state is None else np.asarray(state, dtype=np.float64)
    y = np.zeros_like(x)
    fin = np.zeros((len(segs), 3, C))
    for n, (b, bos, eos) in enumerate(segs):
        ext = np.concatenate([st0[n] if st0 is not None else np.zeros((3, C)), x[b, bos:eos]], axis=0)
        for t in range(eos - bos):
            acc = (w * ext[t:t + 4].T).sum(-1)          # window x[t-3 .. t]
            y[b, bos + t] = acc / (1.0 + np.exp(-acc)) if activation else acc
        fin[n] = ext[-3:]
    return y, fin


def short_conv_backward(x, w, dy, state=None, d_final=None, cu_seqlens=None, activation=False):
    """Reverse-mode gradient of ``short_conv`` (float64) for the loss
    sum <dy, y> + sum <d_final, final state>. Per sequence, with ext the
    window [state; x] (ext[e + 3] = x[e], e >= -3) and p[t] = sum_i w[:, i]
    ext[t + i] the pre-activation:

        dp[t] = dy[t] * (s + p s (1 - s)), s = sigmoid(p[t])   (dy[t] without activation)
        dext[e] = sum_i w[:, i] dp[e - i]  over 0 <= e - i < len    (the transposed taps)
        dext[len + j] += d_final[j]  for the last three window entries (j = 0, 1, 2)
        dw[:, i] = sum over tokens of dp[t] ext[t + i]

    and dext splits into dx (e >= 3) and d_state (e < 3). x, dy [B, T, C];
    w [C, 4]; state, d_final [N, 3, C] or None. Returns (dx [B, T, C],
    dw [C, 4], d_state [N, 3, C]).
    """
    x, w, dy = (np.asarray(a, dtype=np.float64) for a in (x, w, dy))
    B, T, C = x.shape
    segs = _segments(B, T, cu_seqlens)
    st0 = None if state is None else np.asarray(state, dtype=np.float64)
    dfin = None if d_final is None else np.asarray(d_final, dtype=np.float64)
    dx = np.zeros_like(x)
    dw = np.zeros((C, 4))
    dst = np.zeros((len(segs), 3, C))
    for n, (b, bos, eos) in enumerate(segs):
        L = eos - bos
        ext = np.concatenate([st0[n] if st0 is not None else np.zeros((3, C)), x[b, bos:eos]], axis=0)
        dext = np.zeros_like(ext)
        for t in range(L):
            p = (w * ext[t:t + 4].T).sum(-1)
            if activation:
                sg = 1.0 / (1.0 + np.exp(-p))
                dp = dy[b, bos + t] * (sg + p * sg * (1.0 - sg))
            else:
                dp = dy[b, bos + t]
            for i in range(4):
                dext[t + i] += w[:, i] * dp
                dw[:, i] += dp * ext[t + i]
        if dfin is not None:
            dext[L:L + 3] += dfin[n]
        dx[b, bos:eos] = dext[3:]
        dst[n] = dext[:3]
    return dx, dw, dst


def decode_step(q, k, v, g, beta, state_cache, state_slots=None, scale=1.0):
    """One decode step against a state cache. Returns (o [Nb,H,Dv], new cache copy).

    q,k,g: [Nb,H,Dk]; v: [Nb,H,Dv]; beta: [Nb,H]; state_cache [n_slots,H,Dk,Dv];
    row r updates slot state_slots[r] (identity when None). Slots must be distinct.
    """
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    cache = np.array(state_cache, dtype=np.float64)
    Nb = q.shape[0]
    slots = list(range(Nb)) if state_slots is None else [int(s) for s in np.asarray(state_slots)]
    if len(set(slots)) != len(slots):
        raise ValueError("state slots must be distinct")
    o = np.zeros((Nb,) + v.shape[1:])
    for r, s in enumerate(slots):
        S = cache[s]
        o[r] = token_step(S, q[r], k[r], v[r], g[r], beta[r], scale)
    return o, cache


# ----------------------------------------------------------------------------
# C implementation (ctypes)
# ----------------------------------------------------------------------------

_lib = None


def load_c():
    """Load oracle/libkda_ref.so (built by the package build step)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        lib.kda_ref_forward.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I,
                                        ctypes.c_double, P, P, ctypes.c_int]
        lib.kda_ref_forward.restype = ctypes.c_int
        lib.kda_ref_decode_step.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I,
                                            ctypes.c_double, P, ctypes.c_int]
        lib.kda_ref_decode_step.restype = ctypes.c_int
        D = ctypes.c_double
        lib.kda_ref_prologue_forward.argtypes = [P, P, P, P, P, P, P, D, D, P, P, I, I, I, I, I, I,
                                                 D, P, P, ctypes.c_int]
        lib.kda_ref_prologue_forward.restype = ctypes.c_int
        lib.kda_ref_short_conv.argtypes = [P, P, P, P, I, I, I, I, ctypes.c_int, P, P]
        lib.kda_ref_short_conv.restype = ctypes.c_int
        lib.kda_ref_short_conv_step.argtypes = [P, P, P, P, I, I, I, ctypes.c_int, P]
        lib.kda_ref_short_conv_step.restype = ctypes.c_int
        lib.kda_ref_backward.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, D,
                                         P, P, P, P, P, P, ctypes.c_int]
        lib.kda_ref_backward.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def c_forward(q, k, v, g, beta, initial_state=None, cu_seqlens=None, scale=1.0,
              nthreads=0, want_final=True):
    """The C oracle on float32-held inputs. Same contract as ``recurrence``."""
    lib = load_c()
    q, k, v, g, beta = (_f32(a) for a in (q, k, v, g, beta))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    cu = None
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64).reshape(-1))
        N = cu.size - 1
    else:
        N = B
    s0 = None if initial_state is None else _f32(initial_state)
    o = np.zeros((B, T, H, Dv))
    final = np.zeros((N, H, Dk, Dv)) if want_final else None
    rc = lib.kda_ref_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0),
                             _ptr(cu), N, B, T, H, Dk, Dv, float(scale), _ptr(o),
                             _ptr(final), int(nthreads))
    if rc != 0:
        raise ValueError("kda_ref_forward rejected its arguments")
    return o, final


def c_backward(q, k, v, g, beta, d_o, initial_state=None, d_final=None, cu_seqlens=None, scale=1.0,
               nthreads=0):
    """The C oracle's reverse-mode gradient (kda_ref_backward) on float32-held inputs.

    Same contract as ``recurrence_backward``; memory is O(d_k d_v) per token
    block of 64 (forward states re-run from one checkpoint per block).
    """
    lib = load_c()
    q, k, v, g, beta, d_o = (_f32(a) for a in (q, k, v, g, beta, d_o))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    cu = None
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64).reshape(-1))
        N = cu.size - 1
    else:
        N = B
    s0 = None if initial_state is None else _f32(initial_state)
    dfin = None if d_final is None else _f32(d_final)
    dq, dk, dg = (np.zeros((B, T, H, Dk)) for _ in range(3))
    dv = np.zeros((B, T, H, Dv))
    dbeta = np.zeros((B, T, H))
    d_init = np.zeros((N, H, Dk, Dv))
    rc = lib.kda_ref_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0), _ptr(cu),
                              _ptr(d_o), _ptr(dfin), N, B, T, H, Dk, Dv, float(scale),
                              _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(d_init),
                              int(nthreads))
    if rc != 0:
        raise ValueError("kda_ref_backward rejected its arguments")
    return dq, dk, dv, dg, dbeta, d_init


def c_prologue_forward(q_raw, k_raw, v, g_logit, beta_logit, A_log, dt_bias, gate_lower_bound=-5.0,
                       l2_eps=1e-6, initial_state=None, cu_seqlens=None, scale=1.0, nthreads=0,
                       want_final=True):
    """The C oracle from the raw projections: the prologue (see ``prologue``)
    then the recurrence, all in float64."""
    lib = load_c()
    q_raw, k_raw, v, g_logit, beta_logit = (_f32(a) for a in (q_raw, k_raw, v, g_logit, beta_logit))
    A_log, dt_bias = _f32(A_log).reshape(-1), _f32(dt_bias).reshape(-1)
    B, T, H, Dk = q_raw.shape
    Dv = v.shape[-1]
    if A_log.size != Dk or dt_bias.size != H * Dk:
        raise ValueError("A_log must have Dk entries and dt_bias H*Dk")
    cu = None
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64).reshape(-1))
        N = cu.size - 1
    else:
        N = B
    s0 = None if initial_state is None else _f32(initial_state)
    o = np.zeros((B, T, H, Dv))
    final = np.zeros((N, H, Dk, Dv)) if want_final else None
    rc = lib.kda_ref_prologue_forward(_ptr(q_raw), _ptr(k_raw), _ptr(v), _ptr(g_logit), _ptr(beta_logit),
                                      _ptr(A_log), _ptr(dt_bias), float(gate_lower_bound), float(l2_eps),
                                      _ptr(s0), _ptr(cu), N, B, T, H, Dk, Dv, float(scale), _ptr(o),
                                      _ptr(final), int(nthreads))
    if rc != 0:
        raise ValueError("kda_ref_prologue_forward rejected its arguments")
    return o, final


def c_short_conv(x, w, state=None, cu_seqlens=None, activation=False):
    """The C oracle's short convolution (same contract as ``short_conv``)."""
    lib = load_c()
    x, w = _f32(x), _f32(w)
    B, T, C = x.shape
    cu = None
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64).reshape(-1))
        N = cu.size - 1
    else:
        N = B
    st = None if state is None else _f32(state)
    y = np.zeros((B, T, C))
    fin = np.zeros((N, 3, C))
    if lib.kda_ref_short_conv(_ptr(x), _ptr(w), _ptr(st), _ptr(cu), N, B, T, C, int(bool(activation)),
                              _ptr(y), _ptr(fin)) != 0:
        raise ValueError("kda_ref_short_conv rejected its arguments")
    return y, fin


def c_short_conv_step(x, w, cache, slots=None, activation=False):
    """One decode step of the C oracle's convolution; ``cache`` (float64
    [n_slots, 3, C], C-contiguous) is updated in place. Returns y [Nb, C]."""
    lib = load_c()
    if cache.dtype != np.float64 or not cache.flags["C_CONTIGUOUS"]:
        raise TypeError("cache must be a C-contiguous float64 array")
    x, w = _f32(x), _f32(w)
    Nb, C = x.shape
    sl = None if slots is None else np.ascontiguousarray(np.asarray(slots, dtype=np.int64))
    y = np.zeros((Nb, C))
    if lib.kda_ref_short_conv_step(_ptr(x), _ptr(w), _ptr(cache), _ptr(sl), cache.shape[0], Nb, C,
                                   int(bool(activation)), _ptr(y)) != 0:
        raise ValueError("kda_ref_short_conv_step rejected its arguments")
    return y


def c_decode_step(q, k, v, g, beta, state_cache, state_slots=None, scale=1.0, nthreads=0):
    """The C oracle's decode step. ``state_cache`` (float64, C-contiguous) is updated in place."""
    lib = load_c()
    if state_cache.dtype != np.float64 or not state_cache.flags["C_CONTIGUOUS"]:
        raise TypeError("state_cache must be a C-contiguous float64 array")
    q, k, v, g, beta = (_f32(a) for a in (q, k, v, g, beta))
    Nb, H, Dk = q.shape
    Dv = v.shape[-1]
    slots = None
    if state_slots is not None:
        slots = np.ascontiguousarray(np.asarray(state_slots, dtype=np.int64))
    o = np.zeros((Nb, H, Dv))
    rc = lib.kda_ref_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                 _ptr(state_cache), _ptr(slots), state_cache.shape[0],
                                 Nb, H, Dk, Dv, float(scale), _ptr(o), int(nthreads))
    if rc != 0:
        raise ValueError("kda_ref_decode_step rejected its arguments")
    return o


def rel_l2(x, ref):
    """||x - ref||_2 / ||ref||_2 in float64 over whole tensors (absolute L2 when ||ref|| < 1e-30)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = float(np.linalg.norm((x - ref).ravel()))
    den = float(np.linalg.norm(ref.ravel()))
    return num if den < 1e-30 else num / den
