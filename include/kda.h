/*
 * kda.h — C ABI of libkda.so: Kimi Delta Attention (KDA) forward on AMD
 * Instinct MI355X (gfx950).
 *
 * KDA is the gated delta rule with a per-channel diagonal decay. For one
 * sequence and one head, with a state S of d_k x d_v, token t computes
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t
 * It is 69 of the 93 layers of the Kimi K3 text backbone (ISEEKYAN/k3 README,
 * package scope; hysenlabs "kimi-k3-mlx", section "Attention is 93 layers
 * split between KDA and a NoPE gated MLA": 96 heads, head_dim 128). The
 * log-decay g is per token, head AND key channel, a (B,T,96,128) tensor
 * (hysenlabs "kimi-k3-mlx", section "The A_log shape mismatch is a
 * silent-garbage bug the tests assert"), bounded below by gate_lower_bound
 * = -5.0 (section "Attention is 93 layers ...").
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE pointers, row-major and contiguous, owned
 *    by the caller. The library never allocates or frees, and no call but
 *    kda_device_check synchronises; work is enqueued on `stream` (a
 *    hipStream_t; NULL = the default stream) and the call returns before it
 *    finishes.
 *  - Every argument check happens on the host before anything is launched;
 *    a rejected call touches no memory. Unsupported inputs fail explicitly
 *    (the K3 README's rule for unsupported inputs); nothing falls back to
 *    another code path silently.
 *  - g in [-5, 0] (the K3 gate bound). The bf16 matrix-core forward needs
 *    every 16-row chunk's total log-decay per channel, the sum of its 16 g,
 *    in [-84, 0] (g in [-5, 0] keeps it at or above -80) to keep its
 *    in-chunk exponents within float32, and checks that on the device. The
 *    matrix-core backward needs g in [-5, 0] element by element and checks
 *    that. A call that fails either check (a NaN g included) makes the next
 *    kda_device_check return KDA_ERR_DEVICE, and its outputs are not valid.
 *    The other kernels take any finite g.
 *  - Preconditions that are NOT checked on the device: finite inputs,
 *    cu_seqlens starting at 0, non-decreasing and ending at T, distinct
 *    decode state slots.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1, /* NULL pointer, bad size, inconsistent shapes      */
    KDA_ERR_UNSUPPORTED = 2, /* legal but not built: dims, chunk size, dtype     */
    KDA_ERR_HIP = 3,         /* the HIP runtime reported an error at launch      */
    KDA_ERR_DEVICE = 4       /* kda_device_check: a kernel's bounded wait gave up */
} kda_status;

typedef enum {
    KDA_F32 = 0,  /* q,k,v,g,beta and o are float32                             */
    KDA_BF16 = 1  /* q,k,v,g,beta and o are bfloat16; states are always float32  */
} kda_dtype;

/*
 * Chunkwise-parallel KDA forward over whole sequences.
 *
 *   q, k, g        [B,T,H,Dk]  dtype; g is the natural-log decay (decay = exp g)
 *   v              [B,T,H,Dv]  dtype
 *   beta           [B,T,H]     dtype
 *   initial_state  [N,H,Dk,Dv] float32 (Dv contiguous), or NULL for zeros
 *   cu_seqlens     [N+1] int32 offsets of N packed sequences along T (B must be
 *                  1), or NULL: then N must equal B and row b is sequence b.
 *                  Zero-length sequences are allowed: their final state equals
 *                  their initial state. Packed ("THD") batches are how the K3
 *                  package feeds variable-length sequences (ISEEKYAN/k3 README,
 *                  packed THD with context parallelism). The bf16 matrix-core
 *                  kernel starts the longest sequence of each run of 256
 *                  consecutive sequences first (scheduling only: results do
 *                  not depend on it).
 *   chunk_size     0 for the kernel's own chunk length, or an explicit
 *                  length. It changes only rounding. The bf16 matrix-core
 *                  kernel (Dk = Dv = 128) works in 16-row chunks only: there
 *                  chunk_size must be 0 or 16, and any other value is
 *                  KDA_ERR_UNSUPPORTED. The float32 kernel takes
 *                  16, 32 or 64 (0 = 16, its fastest).
 *   scale          multiplies the output (1.0 reproduces the rule above)
 *   o              [B,T,H,Dv]  dtype, written for every row of every sequence;
 *                  must not alias an input. With T = 0, q, k, v, g, beta and
 *                  o may be NULL (only final states are written).
 *   final_state    [N,H,Dk,Dv] float32, or NULL (not written); may alias
 *                  initial_state (each state tile is read before it is written)
 *
 * Supported: Dk, Dv in {16, 32, 64, 128}. bf16 with Dk = Dv = 128 runs the
 * matrix-core kernel; everything else runs the float32 chunk
 * kernel. Chunks start at each sequence's first token; rows
 * past a sequence's end inside its last chunk are treated as zero tokens,
 * which leave the state unchanged.
 */
kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const float* initial_state,
                         const int32_t* cu_seqlens, int32_t B, int32_t T, int32_t H,
                         int32_t Dk, int32_t Dv, int32_t N, int32_t chunk_size, float scale,
                         kda_dtype dtype, void* o, float* final_state, void* stream);

/*
 * Chunkwise KDA forward from the raw projections, with the gate, beta and
 * normalisation prologue computed inside the chunk kernel (no separate pass
 * over HBM). Per token t and head h:
 *   q = q_raw / sqrt(|q_raw|^2 + l2_eps)          over the Dk channels; k likewise
 *   g[c] = gate_lower_bound * sigmoid(exp(A_log[c]) * (g_logit[c] + dt_bias[h*Dk + c]))
 *   beta = sigmoid(beta_logit)
 * then the recurrence of kda_chunk_fwd. The pages give the gate's parameters
 * and bound: A_log has one entry per key channel and is shared by every head,
 * dt_bias one per (head, channel) (hysenlabs "kimi-k3-mlx", section "The A_log
 * shape mismatch is a silent-garbage bug the tests assert"), and
 * gate_lower_bound is -5.0 (section "Attention is 93 layers split between KDA
 * and a NoPE gated MLA"). The formula above is this library's reading of them;
 * the pages do not print it.
 *
 *   q_raw, k_raw, g_logit  [B,T,H,Dk] dtype
 *   v [B,T,H,Dv], beta_logit [B,T,H]  dtype
 *   A_log      [Dk] float32, device;  dt_bias [H*Dk] float32, device
 *   gate_lower_bound  finite and < 0; the gate lies in [gate_lower_bound, 0)
 *   l2_eps     finite and > 0 (rows of zeros normalise to zeros)
 * All other arguments, the ownership rules and the errors are those of
 * kda_chunk_fwd; a bad A_log/dt_bias pointer, bound or eps is
 * KDA_ERR_INVALID_ARG. bf16 with Dk = Dv = 128 and gate_lower_bound >= -5 runs
 * the matrix-core kernel (which relies on g >= -5); everything else runs the
 * float32 chunk kernel. Rows past a sequence's end are zero tokens with g = 0
 * and beta = 0, as in kda_chunk_fwd.
 */
kda_status kda_chunk_fwd_prologue(const void* q_raw, const void* k_raw, const void* v,
                                  const void* g_logit, const void* beta_logit, const float* A_log,
                                  const float* dt_bias, float gate_lower_bound, float l2_eps,
                                  const float* initial_state, const int32_t* cu_seqlens, int32_t B,
                                  int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t N,
                                  int32_t chunk_size, float scale, kda_dtype dtype, void* o,
                                  float* final_state, void* stream);

/*
 * The gate, beta and normalisation prologue of kda_chunk_fwd_prologue on its
 * own: per token and head,
 *   q = q_raw / sqrt(|q_raw|^2 + l2_eps), k likewise,
 *   g = gate_lower_bound * sigmoid(exp(A_log) * (g_logit + dt_bias)),
 *   beta = sigmoid(beta_logit),
 * written in dtype (the parameters and their shapes as cited at
 * kda_chunk_fwd_prologue). It prepares inputs for the calls that take them
 * ready (kda_chunk_fwd, kda_chunk_fwd_split, kda_recurrent_step), for
 * callers that keep them or feed them elsewhere; the fused calls compute the
 * same values inside their kernels (in float32, without rounding them to
 * dtype in between).
 *
 *   q_raw, k_raw, g_logit [B,T,H,Dk], beta_logit [B,T,H]  dtype
 *   A_log [Dk], dt_bias [H*Dk] float32; gate_lower_bound finite and < 0;
 *   l2_eps finite and > 0
 *   q, k, g [B,T,H,Dk], beta [B,T,H]  dtype outputs; each may be its own
 *   input (in place, e.g. q == q_raw) and must not alias anything else
 * T = 0 is a no-op. Errors: KDA_ERR_INVALID_ARG for NULL pointers, bad sizes,
 * bound, eps or aliasing; KDA_ERR_UNSUPPORTED for dims outside
 * {16, 32, 64, 128} or another dtype.
 */
kda_status kda_prologue(const void* q_raw, const void* k_raw, const void* g_logit, const void* beta_logit,
                        const float* A_log, const float* dt_bias, float gate_lower_bound, float l2_eps, int32_t B,
                        int32_t T, int32_t H, int32_t Dk, kda_dtype dtype, void* q, void* k, void* g, void* beta,
                        void* stream);

/*
 * Bytes of device workspace kda_chunk_fwd_conv needs (0 for T = 0 or
 * out-of-range sizes): for bf16 with Dk = Dv = 128 and gate_lower_bound >= -5
 * (v convolved in the chunk kernel) the convolved q and k, 2 x B*T*H*Dk bf16; otherwise the
 * three convolved projections, B*T*H*(2 Dk + Dv) elements of dtype.
 */
size_t kda_chunk_fwd_conv_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, kda_dtype dtype,
                                          float gate_lower_bound);

/*
 * The KDA layer's token mixer from the projections before the short
 * convolution: for each of q, k and v the kernel-4 causal convolution of
 * kda_short_conv (with its conv state and optional SiLU; K3 runs a short
 * convolution of kernel size 4 on the query, key and value projections before
 * KDA: hysenlabs "kimi-k3-mlx", section "Attention is 93 layers split between
 * KDA and a NoPE gated MLA"), its output rounded to dtype, then
 * kda_chunk_fwd_prologue on the convolved q, k and v. The result equals that
 * sequence of calls (bit for bit on the fused path).
 *
 * For bf16 with Dk = Dv = 128 and gate_lower_bound >= -5, the convolution of
 * v runs inside the chunk kernel: its state waves, idle for part of every
 * group, convolve each group of v in registers as it arrives (the convolved v
 * never goes to memory); q and k are convolved into the workspace by the
 * streaming convolution kernel first. Every other supported shape runs the
 * three convolutions into the workspace, then the prologue forward.
 *
 *   xq, xk [B,T,H,Dk], xv [B,T,H,Dv]  dtype: the projections before the convolution
 *   wq, wk [H*Dk][4], wv [H*Dv][4]     float32 taps (16-byte aligned rows)
 *   conv_state_q, _k, _v  [N][3][H*D] float32 (x[-3], x[-2], x[-1] of each
 *                          sequence), or NULL for zeros
 *   activation             0 = none, 1 = SiLU after each convolution
 *   g_logit, beta_logit, A_log, dt_bias, gate_lower_bound, l2_eps, initial_state,
 *   cu_seqlens, B, T, H, Dk, Dv, N, chunk_size, scale, dtype, o, final_state
 *                          as for kda_chunk_fwd_prologue
 *   workspace              at least kda_chunk_fwd_conv_workspace_bytes(...) bytes
 *                          of device memory, not overlapping any input or output;
 *                          contents on entry do not matter
 *   conv_state_q_out, _k_out, _v_out  [N][3][H*D] float32 or NULL: each
 *                          sequence's last three inputs (as kda_short_conv's
 *                          conv_state_out; may alias the input states)
 * Errors as for kda_chunk_fwd_prologue and kda_short_conv; NULL taps, a bad
 * activation or a short workspace are KDA_ERR_INVALID_ARG.
 */
kda_status kda_chunk_fwd_conv(const void* xq, const void* xk, const void* xv, const float* wq, const float* wk,
                              const float* wv, const float* conv_state_q, const float* conv_state_k,
                              const float* conv_state_v, int32_t activation, const void* g_logit,
                              const void* beta_logit, const float* A_log, const float* dt_bias,
                              float gate_lower_bound, float l2_eps, const float* initial_state,
                              const int32_t* cu_seqlens, int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv,
                              int32_t N, int32_t chunk_size, float scale, kda_dtype dtype, void* workspace,
                              size_t workspace_bytes, void* o, float* final_state, float* conv_state_q_out,
                              float* conv_state_k_out, float* conv_state_v_out, void* stream);

/*
 * Bytes of device workspace kda_chunk_fwd_split needs for these sizes and
 * segments >= 2 (0 for segments <= 1, T = 0 or out-of-range sizes; the same
 * for packed and fixed-length batches with the same N).
 */
size_t kda_chunk_fwd_split_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t N,
                                           kda_dtype dtype, int32_t segments);

/*
 * kda_chunk_fwd with every sequence cut into `segments` pieces that run in
 * parallel, for batches with too few (sequence, head) pairs to fill the chip
 * (a long sequence over few heads, as one GPU's share of a head-sharded
 * layer). The package the method comes from notes that context parallelism is
 * not available on its first KDA path and feeds long inputs as packed THD with
 * context parallelism (ISEEKYAN/k3 README); this is the same idea inside one
 * GPU. Over a segment the recurrence is affine in its entry state,
 * S_out = A S_in + B (B: the final state from a zero entry state; A, d_k x d_k:
 * from the identity with v = 0), and so is every row's state, so a row's
 * output is its output from a zero entry state plus S_inᵀ (scale A_tᵀ q_t).
 *   bf16, d_k = d_v = 128: one launch runs B over every segment (a sequence's
 *   first segment from its initial state, so its outputs are final) and A
 *   over the others, keeping A's outputs; a scan chains the entry states
 *   S_in(p) = A(p-1) S_in(p-1) + B(p-1) per sequence; a last kernel adds the
 *   correction to the rows of segments after the first.
 *   Other shapes: the forward over all segments from zero states (B), again
 *   with v = 0 from identity states (A), the scan, and the forward over all
 *   segments once more from S_in, which writes o.
 *
 * Segments are cut at multiples of 64 rows. With s = roundup(ceil(L/(segments
 * + w - 1)), 64) for a sequence of length L, the first segment takes w * s
 * rows and each later one s rows, the last shorter and trailing ones possibly
 * empty; w = 2 on the bf16 d_k = d_v = 128 path (its first segments run one
 * pass, the others two), 1 otherwise. The results equal kda_chunk_fwd's up to
 * rounding (the entry states carry the rounding of A and B).
 *
 *   segments   1 .. 4096; 1 (or T = 0) runs kda_chunk_fwd and needs no
 *              workspace
 *   workspace  at least kda_chunk_fwd_split_workspace_bytes(...) bytes of
 *              device memory owned by the caller, not overlapping any input or
 *              output; its contents on entry do not matter
 * All other arguments, the supported shapes and the errors are those of
 * kda_chunk_fwd; B*T must fit in int32. A short or NULL workspace is
 * KDA_ERR_INVALID_ARG.
 */
kda_status kda_chunk_fwd_split(const void* q, const void* k, const void* v, const void* g, const void* beta,
                               const float* initial_state, const int32_t* cu_seqlens, int32_t B, int32_t T,
                               int32_t H, int32_t Dk, int32_t Dv, int32_t N, int32_t chunk_size, float scale,
                               kda_dtype dtype, int32_t segments, void* workspace, size_t workspace_bytes, void* o,
                               float* final_state, void* stream);

/*
 * kda_chunk_fwd_split from raw projections: the gate, beta and normalisation
 * prologue of kda_chunk_fwd_prologue inside every pass of the split, for long
 * sequences of a layer whose inputs are the projections (the K3 layer's
 * parameters as cited at kda_chunk_fwd_prologue). q_raw, k_raw, v, g_logit,
 * beta_logit, A_log, dt_bias, gate_lower_bound and l2_eps as for
 * kda_chunk_fwd_prologue; segments, workspace (at least
 * kda_chunk_fwd_split_workspace_bytes for the same sizes) and the rest as for
 * kda_chunk_fwd_split. bf16 with Dk = Dv = 128 and gate_lower_bound >= -5 runs
 * the matrix-core form, everything else the float32 passes. Errors as for
 * both.
 */
kda_status kda_chunk_fwd_split_prologue(const void* q_raw, const void* k_raw, const void* v, const void* g_logit,
                                        const void* beta_logit, const float* A_log, const float* dt_bias,
                                        float gate_lower_bound, float l2_eps, const float* initial_state,
                                        const int32_t* cu_seqlens, int32_t B, int32_t T, int32_t H, int32_t Dk,
                                        int32_t Dv, int32_t N, int32_t chunk_size, float scale, kda_dtype dtype,
                                        int32_t segments, void* workspace, size_t workspace_bytes, void* o,
                                        float* final_state, void* stream);

/*
 * kda_chunk_fwd_split for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. Identical to kda_chunk_fwd_split (same arguments minus the
 * workspace, same kernels, same results), except that the workspace is the
 * library's static scratch: a device array of KDA_SPLIT_STATIC_SCRATCH_BYTES
 * that every device the library runs on holds from module load until the
 * process ends. The call allocates and frees nothing.
 *
 *   Sizes whose kda_chunk_fwd_split_workspace_bytes exceeds
 *   KDA_SPLIT_STATIC_SCRATCH_BYTES are KDA_ERR_UNSUPPORTED (before any launch).
 *   Every call on a device shares that device's scratch and leaves its last
 *   contents in it (no call needs it to start at zero). Calls that overlap in
 *   time on one device (from several streams or threads) race on it and give
 *   undefined results: serialise them, e.g. on one stream.
 */
#define KDA_SPLIT_STATIC_SCRATCH_BYTES ((size_t)128 << 20)
kda_status kda_chunk_fwd_split_static(const void* q, const void* k, const void* v, const void* g,
                                      const void* beta, const float* initial_state, const int32_t* cu_seqlens,
                                      int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t N,
                                      int32_t chunk_size, float scale, kda_dtype dtype, int32_t segments, void* o,
                                      float* final_state, void* stream);

/*
 * Bytes of device workspace kda_chunk_bwd needs: per 16-row chunk slot and
 * head, one float32 state [Dk,Dv] plus three float32 16x16 matrices; T/16 + N
 * slots for packed sequences (packed != 0), B * ceil(T/16) otherwise. 0 when
 * T = 0 or a size is out of range.
 */
size_t kda_chunk_bwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t N,
                                     int32_t packed);

/*
 * Backward of kda_chunk_fwd: the gradients of
 *   L = sum_t <d_o[t], o[t]> + sum_n <d_final_state[n], final_state[n]>
 * with respect to q, k, v, g, beta and initial_state, for the recurrence and
 * the scale that kda_chunk_fwd computes. The package the method comes from
 * trains through KDA (ISEEKYAN/k3 README: its single-rank reference path runs
 * a KDA layer through loss and backward), while the FlashKDA backend it names
 * is forward-only; this is the training-side counterpart of the forward here.
 *
 *   q, k, v, g, beta, initial_state, cu_seqlens, B, T, H, Dk, Dv, N, scale,
 *   dtype     exactly as passed to kda_chunk_fwd
 *   d_o       [B,T,H,Dv] dtype: gradient of the loss with respect to o
 *   d_final_state  [N,H,Dk,Dv] float32, or NULL for zeros
 *   workspace at least kda_chunk_bwd_workspace_bytes(...) bytes of device
 *             memory (packed = cu_seqlens != NULL), owned by the caller; its
 *             contents on entry do not matter and are overwritten (the
 *             forward's state at the start of every 16-row chunk)
 *   dq, dk, dg [B,T,H,Dk], dv [B,T,H,Dv], dbeta [B,T,H]: float32 outputs,
 *             written for every row of every sequence; they must not alias
 *             an input or the workspace
 *   d_initial_state [N,H,Dk,Dv] float32, or NULL (not written)
 *
 * Everything is computed in float32, in 16-row chunks; bf16 inputs are
 * widened exactly. Dk = 128 with Dv = 64 or 128 runs a matrix-core kernel
 * (float32 MFMA) that factors the in-chunk decay through the chunk's middle
 * row and so relies on g in [-5, 0], which it checks on the device like the
 * forward (kda_device_check reports a g outside it); other head
 * dims run a vector-ALU kernel with no range condition on g. For Dv = 128 the two 64-column halves of
 * the value dimension add their shares of dq, dk, dg and dbeta with float32
 * atomics, which with two terms is order-independent, so the result is
 * deterministic. With T = 0 only d_initial_state is written (it then equals
 * d_final_state, or zeros). Supported dims and errors as for kda_chunk_fwd; a
 * short or NULL workspace is KDA_ERR_INVALID_ARG.
 */
kda_status kda_chunk_bwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                         const float* initial_state, const int32_t* cu_seqlens, const void* d_o,
                         const float* d_final_state, int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv,
                         int32_t N, float scale, kda_dtype dtype, void* workspace, size_t workspace_bytes,
                         float* dq, float* dk, float* dv, float* dg, float* dbeta, float* d_initial_state,
                         void* stream);

/*
 * Bytes of device workspace kda_chunk_bwd_prologue needs: that of
 * kda_chunk_bwd for the same sizes, plus float32 copies of the prologue's
 * outputs (q, k, g [B,T,H,Dk], beta [B,T,H]) and room for float32 copies of v
 * and d_o [B,T,H,Dv] (written only when bf16 inputs go to the vector-ALU
 * backward), plus 2 x ceil(B*T/64) x H x Dk floats of partial sums. 0 when
 * T = 0 or a size is out of range.
 */
size_t kda_chunk_bwd_prologue_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t N,
                                              int32_t packed);

/*
 * Backward of kda_chunk_fwd_prologue: the gradients of
 *   L = sum_t <d_o[t], o[t]> + sum_n <d_final_state[n], final_state[n]>
 * with respect to the raw projections q_raw, k_raw, g_logit, beta_logit, to v,
 * to the gate parameters A_log and dt_bias, and to initial_state. The prologue
 * (the reading documented with kda_chunk_fwd_prologue) is differentiated line
 * by line:
 *   q = x / n, n = sqrt(|x|^2 + eps):  dx = dq / n - x (x . dq) / n^3   (k likewise)
 *   g = lb s, s = sigmoid(z), z = exp(A_log[c]) (g_logit + dt_bias[h,c]):
 *     dz = dg lb s (1 - s), d g_logit = dz exp(A_log[c]),
 *     d dt_bias[h,c] = sum over tokens of dz exp(A_log[c]),
 *     d A_log[c] = sum over tokens and heads of dz z
 *   beta = sigmoid(y):  dy = dbeta beta (1 - beta)
 * around kda_chunk_bwd's gradient of the recurrence. The K3 gate's
 * parameters are trained with the layer (they are checkpoint weights:
 * hysenlabs "kimi-k3-mlx", section "The A_log shape mismatch is a
 * silent-garbage bug the tests assert").
 *
 *   inputs     as kda_chunk_fwd_prologue (same dtype for the raw projections,
 *              v and d_o), with d_o and d_final_state as in kda_chunk_bwd
 *   workspace  at least kda_chunk_bwd_prologue_workspace_bytes(...) bytes,
 *              owned by the caller; contents on entry do not matter
 *   dq_raw, dk_raw, dg_logit [B,T,H,Dk], dv [B,T,H,Dv], dbeta_logit [B,T,H],
 *   dA_log [Dk], ddt_bias [H*Dk], d_initial_state [N,H,Dk,Dv] (or NULL):
 *              float32 outputs; must not alias an input or the workspace
 *
 * The recurrence's part runs on float32 copies of the prologue's outputs, so
 * every step is float32 (kda_chunk_bwd's matrix-core kernel for Dk = 128 and
 * gate_lower_bound >= -5, its vector-ALU kernel otherwise).
 * dA_log and ddt_bias are summed in a fixed order and the call is
 * deterministic. Errors as for kda_chunk_bwd; a NULL A_log, dt_bias, dA_log
 * or ddt_bias, a non-negative or non-finite gate_lower_bound or a
 * non-positive l2_eps is KDA_ERR_INVALID_ARG.
 */
kda_status kda_chunk_bwd_prologue(const void* q_raw, const void* k_raw, const void* v, const void* g_logit,
                                  const void* beta_logit, const float* A_log, const float* dt_bias,
                                  float gate_lower_bound, float l2_eps, const float* initial_state,
                                  const int32_t* cu_seqlens, const void* d_o, const float* d_final_state, int32_t B,
                                  int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t N, float scale,
                                  kda_dtype dtype, void* workspace, size_t workspace_bytes, float* dq_raw,
                                  float* dk_raw, float* dv, float* dg_logit, float* dbeta_logit, float* dA_log,
                                  float* ddt_bias, float* d_initial_state, void* stream);

/*
 * Bytes of device workspace kda_chunk_bwd_conv needs: the three recomputed
 * convolution outputs (dtype) and their float32 gradients, B*T*H*(2 Dk + Dv)
 * elements each, plus the larger of kda_chunk_bwd_prologue_workspace_bytes
 * and kda_short_conv_bwd_workspace_bytes for the same sizes (each 256-byte
 * aligned). 0 when T = 0 or a size is out of range.
 */
size_t kda_chunk_bwd_conv_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t N,
                                          int32_t packed, kda_dtype dtype);

/*
 * Backward of kda_chunk_fwd_conv: the gradients of
 *   L = sum_t <d_o[t], o[t]> + sum_n <d_final_state[n], final_state[n]>
 *       + sum_n sum_j <d_conv_final_j[n], conv_state_j_out[n]>   (j = q, k, v)
 * with respect to the projections before the short convolution, the taps,
 * the initial conv states, the gate logits and parameters and the initial
 * state. It recomputes the three convolutions into the workspace, runs
 * kda_chunk_bwd_prologue on them, then kda_short_conv_bwd for each projection
 * (the convolution before the prologue: hysenlabs "kimi-k3-mlx", section
 * "Attention is 93 layers split between KDA and a NoPE gated MLA"), and
 * equals that sequence of calls bit for bit. This is the layer's backward for
 * training from the pre-convolution projections (ISEEKYAN/k3 README, the
 * single-rank reference path that runs loss and backward).
 *
 *   xq, xk, xv, wq, wk, wv, conv_state_q, _k, _v, activation, g_logit, beta_logit,
 *   A_log, dt_bias, gate_lower_bound, l2_eps, initial_state, cu_seqlens,
 *   B, T, H, Dk, Dv, N, scale, dtype
 *                 exactly as passed to kda_chunk_fwd_conv
 *   d_o, d_final_state
 *                 as for kda_chunk_bwd
 *   d_conv_final_q, _k, _v  [N][3][H*D] float32 or NULL (zeros): cotangents
 *                 of the final conv states
 *   workspace     at least kda_chunk_bwd_conv_workspace_bytes(...) bytes,
 *                 owned by the caller; contents on entry do not matter
 *   dxq, dxk [B,T,H,Dk], dxv [B,T,H,Dv]; dwq, dwk [H*Dk][4], dwv [H*Dv][4];
 *   d_conv_state_q, _k, _v [N][3][H*D] (or NULL, not written); dg_logit,
 *   dbeta_logit, dA_log, ddt_bias, d_initial_state (or NULL) as for
 *   kda_chunk_bwd_prologue: float32 outputs that must not alias an input
 *
 * Errors as for kda_chunk_bwd_prologue and kda_short_conv_bwd (their messages
 * are prefixed with this call's name); NULL or misaligned taps, a NULL tap
 * gradient or a bad activation are KDA_ERR_INVALID_ARG.
 */
kda_status kda_chunk_bwd_conv(const void* xq, const void* xk, const void* xv, const float* wq, const float* wk,
                              const float* wv, const float* conv_state_q, const float* conv_state_k,
                              const float* conv_state_v, int32_t activation, const void* g_logit,
                              const void* beta_logit, const float* A_log, const float* dt_bias,
                              float gate_lower_bound, float l2_eps, const float* initial_state,
                              const int32_t* cu_seqlens, const void* d_o, const float* d_final_state,
                              const float* d_conv_final_q, const float* d_conv_final_k,
                              const float* d_conv_final_v, int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv,
                              int32_t N, float scale, kda_dtype dtype, void* workspace, size_t workspace_bytes,
                              float* dxq, float* dxk, float* dxv, float* dwq, float* dwk, float* dwv,
                              float* d_conv_state_q, float* d_conv_state_k, float* d_conv_state_v,
                              float* dg_logit, float* dbeta_logit, float* dA_log, float* ddt_bias,
                              float* d_initial_state, void* stream);

/*
 * Short causal depthwise convolution over time (kernel size 4), the step that
 * KDA applies to the query, key and value projections before the recurrence
 * (hysenlabs "kimi-k3-mlx", section "Attention is 93 layers split between KDA
 * and a NoPE gated MLA"; the pages give the kernel size only, the formula below
 * is this library's reading). Per sequence and channel c:
 *   y[t][c] = sum_{i=0..3} weight[c][i] * x[t - 3 + i][c]
 * with the three inputs before a sequence's first token taken from
 * conv_state_in, then y <- y * sigmoid(y) when activation = 1. Call it once per
 * projection (q, k, v: C = H*Dk or H*Dv channels, the [B,T,H,D] tensor viewed
 * as [B,T,C]).
 *
 *   x               [B,T,C] dtype; y [B,T,C] dtype, must not alias x
 *   weight          [C][4] float32 (16-byte aligned rows)
 *   conv_state_in   [N][3][C] float32: x[-3], x[-2], x[-1] of each sequence,
 *                   or NULL for zeros
 *   conv_state_out  [N][3][C] float32, or NULL: the last three inputs of each
 *                   sequence's window (reaching into conv_state_in when a
 *                   sequence has fewer than 3 tokens); may alias conv_state_in
 *   cu_seqlens      as for kda_chunk_fwd (packed sequences, B = 1), or NULL
 *   activation      0 = none, 1 = SiLU
 * Supported: C a multiple of 8; dtype KDA_F32 or KDA_BF16. Errors as for
 * kda_chunk_fwd.
 */
kda_status kda_short_conv(const void* x, const float* weight, const float* conv_state_in,
                          const int32_t* cu_seqlens, int32_t B, int32_t T, int32_t C, int32_t N,
                          int32_t activation, kda_dtype dtype, void* y, float* conv_state_out, void* stream);

/* Bytes of device workspace kda_short_conv_bwd needs: ceil(B*T/256) x C x 4 floats. */
size_t kda_short_conv_bwd_workspace_bytes(int32_t B, int32_t T, int32_t C);

/*
 * Backward of kda_short_conv: the gradients of
 *   L = sum <dy, y> + sum_n <d_final_state[n], conv_state_out[n]>
 * with respect to x, weight and conv_state_in. With p[t] the pre-activation
 * and dp[t] = dy[t] act'(p[t]) (act' = 1 without activation; for SiLU,
 * s + p s (1 - s) with s = sigmoid(p)), per sequence and channel c:
 *   dx[t][c]      = sum_i weight[c][i] dp[t + 3 - i][c]   (terms inside the sequence)
 *                   + d_final_state for the window's last three inputs
 *   dweight[c][i] = sum over all tokens t of dp[t][c] x[t - 3 + i][c]
 *   d_state_in[n][j][c] = sum_{i <= j} weight[c][i] dp[bos + j - i][c]
 *                   (+ d_final_state where a short sequence's final window
 *                   still holds state entries)
 * This is the convolution that sits before the prologue (the reading of the
 * pages documented with kda_short_conv), so it chains after
 * kda_chunk_bwd_prologue: its dq_raw, dk_raw and dv are dy for the three
 * projections.
 *
 *   x, weight, conv_state_in, cu_seqlens, B, T, C, N, activation, dtype
 *              exactly as passed to kda_short_conv
 *   dy         [B,T,C] float32;  d_final_state [N][3][C] float32 or NULL
 *   workspace  at least kda_short_conv_bwd_workspace_bytes(B, T, C) bytes
 *   dx [B,T,C], dweight [C][4] float32 outputs; d_state_in [N][3][C] float32
 *              or NULL (not written); none may alias an input
 * dweight is summed over token blocks in a fixed order, so the call is
 * deterministic. Errors as for kda_short_conv.
 */
kda_status kda_short_conv_bwd(const void* x, const float* weight, const float* conv_state_in,
                              const int32_t* cu_seqlens, const float* dy, const float* d_final_state, int32_t B,
                              int32_t T, int32_t C, int32_t N, int32_t activation, kda_dtype dtype, void* workspace,
                              size_t workspace_bytes, float* dx, float* dweight, float* d_state_in, void* stream);

/*
 * One decode step of the short convolution: row r (one token) reads the three
 * previous inputs from conv_cache[slot(r)] ([3][C] float32), writes
 * y[r] = sum_i weight[c][i] * window[i] (then SiLU if activation = 1) and
 * shifts x[r] into the cache. slot(r) = cache_slots[r], or r when cache_slots
 * is NULL; slots in range must be distinct. A row whose slot lies outside
 * [0, n_slots) (for example -1, a padding row) gets y = 0 and leaves the
 * cache untouched.
 *   x, y [Nb][C] dtype; conv_cache [n_slots][3][C] float32, updated in place.
 * Nb = 0 is a no-op. Errors as for kda_recurrent_step.
 */
kda_status kda_short_conv_step(const void* x, const float* weight, float* conv_cache, const int32_t* cache_slots,
                               int32_t n_slots, int32_t Nb, int32_t C, int32_t activation, kda_dtype dtype,
                               void* y, void* stream);

/*
 * One decode step (T = 1 per row) against a state cache, updated in place:
 * the recurrence above applied to one token per (row, head),
 *   S' = Diag(exp g) S,  u = beta (v - S'^T k),  S <- S' + k u^T,
 *   o = scale * S^T q.
 * This is the step K3 runs for each generated token in its 69 KDA layers
 * (ISEEKYAN/k3 README, package scope: the recurrent KDA layers of the K3
 * backbone; hysenlabs "kimi-k3-mlx", section "Attention is 93 layers split
 * between KDA and a NoPE gated MLA": 96 heads of 128 channels, so 64 KiB of
 * float32 state per head and sequence). The per-channel decay and its bound
 * are those of kda_chunk_fwd.
 *
 *   q, k, g      [Nb,H,Dk] dtype;  v [Nb,H,Dv] dtype;  beta [Nb,H] dtype
 *   state_cache  [n_slots,H,Dk,Dv] float32
 *   state_slots  [Nb] int32 device array: row r reads and writes slot
 *                state_slots[r]; NULL means slot r. Slots in range must be
 *                distinct. A row whose slot lies outside [0, n_slots) (for
 *                example -1, a padding row of a serving batch) is skipped on
 *                the device: its o is zero and no state is read or written.
 *   o            [Nb,H,Dv] dtype
 *
 * Supported: Dk, Dv in {16, 32, 64, 128}. Nb = 0 is a no-op (pointers may
 * then be NULL).
 */
kda_status kda_recurrent_step(const void* q, const void* k, const void* v, const void* g,
                              const void* beta, float* state_cache, const int32_t* state_slots,
                              int32_t n_slots, int32_t Nb, int32_t H, int32_t Dk, int32_t Dv,
                              float scale, kda_dtype dtype, void* o, void* stream);

/*
 * kda_recurrent_step from raw projections: per (row, head) the gate, beta and
 * normalisation prologue of kda_chunk_fwd_prologue (q and k scaled to unit
 * length, g = gate_lower_bound * sigmoid(exp(A_log) * (g_logit + dt_bias)),
 * beta = sigmoid(beta_logit)), then the decode step, in one kernel. This is
 * the per-token form of the prologue forward, for a generation loop that
 * keeps the recurrent state between tokens; the pages' parameters and bound
 * are those cited at kda_chunk_fwd_prologue.
 *
 *   q_raw, k_raw, g_logit  [Nb,H,Dk] dtype;  v [Nb,H,Dv];  beta_logit [Nb,H]
 *   A_log [Dk], dt_bias [H*Dk] float32; gate_lower_bound finite and < 0;
 *   l2_eps finite and > 0
 *   state_cache, state_slots, n_slots, Nb, H, Dk, Dv, scale, dtype, o
 *                as for kda_recurrent_step (padding rows included)
 * The decay factor exp(g) lies in [exp(gate_lower_bound), 1) for any logits,
 * so there is no range precondition. Errors as for kda_recurrent_step; a NULL
 * A_log or dt_bias, a bad bound or eps is KDA_ERR_INVALID_ARG.
 */
kda_status kda_recurrent_step_prologue(const void* q_raw, const void* k_raw, const void* v, const void* g_logit,
                                       const void* beta_logit, const float* A_log, const float* dt_bias,
                                       float gate_lower_bound, float l2_eps, float* state_cache,
                                       const int32_t* state_slots, int32_t n_slots, int32_t Nb, int32_t H,
                                       int32_t Dk, int32_t Dv, float scale, kda_dtype dtype, void* o,
                                       void* stream);

/*
 * One generated token of the KDA layer from the projections before the short
 * convolution (the decode form of kda_chunk_fwd_conv): for each of q, k and v
 * the convolution step of kda_short_conv_step over its cache, its output
 * rounded to dtype, then kda_recurrent_step_prologue on the convolved q, k
 * and v, all in one kernel. The result, the state cache and the three
 * convolution caches equal those of that sequence of calls bit for bit.
 *
 *   xq, xk [Nb,H,Dk], xv [Nb,H,Dv]  dtype: the projections before the convolution
 *   wq, wk [H*Dk][4], wv [H*Dv][4]   float32 taps, 16-byte aligned
 *   conv_cache_q, _k [n_slots][3][H*Dk], conv_cache_v [n_slots][3][H*Dv]
 *                float32, updated in place, indexed by the same slot as the
 *                state cache (a padding row touches none of them)
 *   activation   0 = none, 1 = SiLU after each convolution
 *   the rest     as for kda_recurrent_step_prologue
 * Errors as for kda_recurrent_step_prologue and kda_short_conv_step; NULL or
 * misaligned taps, a NULL cache or a bad activation are KDA_ERR_INVALID_ARG,
 * as is a convolution cache that is the state cache or another's.
 */
kda_status kda_recurrent_step_conv(const void* xq, const void* xk, const void* xv, const float* wq,
                                   const float* wk, const float* wv, float* conv_cache_q, float* conv_cache_k,
                                   float* conv_cache_v, int32_t activation, const void* g_logit,
                                   const void* beta_logit, const float* A_log, const float* dt_bias,
                                   float gate_lower_bound, float l2_eps, float* state_cache,
                                   const int32_t* state_slots, int32_t n_slots, int32_t Nb, int32_t H, int32_t Dk,
                                   int32_t Dv, float scale, kda_dtype dtype, void* o, void* stream);

/*
 * Device-side failures. The bf16 matrix-core forward hands work between the
 * waves of a workgroup through flags in LDS; every wait for such a flag is
 * bounded. A producer always stores its flag, so a wait that gives up means a
 * fault in the library, and the outputs of that call are then not valid.
 * Instead of hanging or returning silently wrong data, the kernel counts
 * each give-up in a per-device status word, finishes normally, and
 * kda_device_check reports it: failures are explicit (ISEEKYAN/k3 README,
 * package scope). A second status word counts log-decays out of the range
 * the matrix-core kernels need (see the conventions above).
 *
 * kda_device_check waits for the work enqueued on `stream`, then returns
 * KDA_OK if, since the previous check (or since the library was loaded), no
 * bounded wait of any call on the current device gave up and no gate fell
 * outside its range, and KDA_ERR_DEVICE otherwise (kda_last_error_message
 * says which, with the count). The check itself synchronises, so it belongs
 * outside timed or captured regions.
 */
kda_status kda_device_check(void* stream);

/*
 * Polls of one bounded wait before it gives up (default 4194304, about 0.1 s
 * of sleeping polls), for every call launched afterwards from any thread.
 * Negative values are KDA_ERR_INVALID_ARG. A limit of 0 makes a wait give up
 * whenever its flag is not already set; that is only useful to exercise the
 * error path of kda_device_check.
 */
kda_status kda_set_wait_limit(int32_t polls);

/* Static name of a status code. */
const char* kda_status_string(kda_status s);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* kda_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
