/*
 * Plain fp64 CPU oracle for Kimi Delta Attention (KDA): the gated delta rule
 * with a per-channel diagonal decay, run one token at a time.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or
 * load this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it. It shares no code with the HIP kernels.
 *
 * What it computes (per sequence n and head h, for t in order):
 *   S <- Diag(exp g_t) S                       decay first, one factor per key channel
 *   S <- S + beta_t k_t (v_t - S^T k_t)^T      = (I - beta_t k_t k_t^T) S + beta_t k_t v_t^T
 *   o_t = scale * S^T q_t                       read from the post-update state
 * This is the gated delta rule of Kimi Delta Attention as the Kimi K3 pages
 * name it (ISEEKYAN/k3 README, KDA compute path; hysenlabs "kimi-k3-mlx",
 * section "The A_log shape mismatch ...": the log-decay g has shape
 * (B,T,96,128), i.e. one value per token, head and key channel).
 *
 * Layouts (row-major, the same as the library's):
 *   q,k,g [B,T,H,Dk]; v [B,T,H,Dv]; beta [B,T,H]; o [B,T,H,Dv]
 *   states [N,H,Dk,Dv] (Dv contiguous); cu_seqlens [N+1] (B must be 1)
 * Inputs are float: bf16 and fp32 values are both held exactly in float and
 * every operation below is carried out in double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One token of the recurrence on one (sequence, head) state S [Dk][Dv]; the
 * token's rows are given in double. */
static void kda_ref_token(double* S, double* x, const double* qt, const double* kt,
                          const double* vt, const double* gt, double bt,
                          int64_t Dk, int64_t Dv, double scale, double* ot)
{
    for (int64_t i = 0; i < Dk; ++i) {
        const double a = exp(gt[i]);
        double* row = S + i * Dv;
        for (int64_t j = 0; j < Dv; ++j) row[j] *= a;
    }
    for (int64_t j = 0; j < Dv; ++j) x[j] = 0.0;
    for (int64_t i = 0; i < Dk; ++i) {
        const double ki = kt[i];
        const double* row = S + i * Dv;
        for (int64_t j = 0; j < Dv; ++j) x[j] += ki * row[j];
    }
    for (int64_t j = 0; j < Dv; ++j) x[j] = bt * (vt[j] - x[j]);
    for (int64_t i = 0; i < Dk; ++i) {
        const double ki = kt[i];
        double* row = S + i * Dv;
        for (int64_t j = 0; j < Dv; ++j) row[j] += ki * x[j];
    }
    if (ot) {
        for (int64_t j = 0; j < Dv; ++j) x[j] = 0.0;
        for (int64_t i = 0; i < Dk; ++i) {
            const double qi = qt[i];
            const double* row = S + i * Dv;
            for (int64_t j = 0; j < Dv; ++j) x[j] += qi * row[j];
        }
        for (int64_t j = 0; j < Dv; ++j) ot[j] = scale * x[j];
    }
}

/* float -> double (exact) */
static void widen(const float* src, double* dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) dst[i] = (double)src[i];
}

/* Row buffers of one token in double: q, k, g [Dk] and v [Dv]. */
typedef struct { double *q, *k, *g, *v, *x; } rows_t;

static int rows_alloc(rows_t* r, int64_t Dk, int64_t Dv)
{
    r->q = (double*)malloc(sizeof(double) * Dk);
    r->k = (double*)malloc(sizeof(double) * Dk);
    r->g = (double*)malloc(sizeof(double) * Dk);
    r->v = (double*)malloc(sizeof(double) * Dv);
    r->x = (double*)malloc(sizeof(double) * Dv);
    return r->q && r->k && r->g && r->v && r->x;
}

static void rows_free(rows_t* r)
{
    free(r->q); free(r->k); free(r->g); free(r->v); free(r->x);
}

/*
 * Forward over whole sequences. Returns 0, or -1 on bad arguments / no memory.
 * o [B,T,H,Dv] (rows outside every sequence are left untouched);
 * final_state [N,H,Dk,Dv] may be NULL. nthreads <= 0 means the OpenMP default.
 */
int kda_ref_forward(const float* q, const float* k, const float* v, const float* g,
                    const float* beta, const float* initial_state,
                    const int64_t* cu_seqlens, int64_t N,
                    int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                    double scale, double* o, double* final_state, int nthreads)
{
    if (!q || !k || !v || !g || !beta || !o || B < 1 || T < 0 || H < 1 || Dk < 1 || Dv < 1)
        return -1;
    if (cu_seqlens) {
        if (B != 1 || N < 1 || cu_seqlens[0] != 0 || cu_seqlens[N] != T) return -1;
        for (int64_t n = 0; n < N; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    } else {
        N = B;
    }
    int failed = 0;
    const int64_t units = N * H;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : failed)
#endif
    for (int64_t u = 0; u < units; ++u) {
        const int64_t n = u / H, h = u % H;
        const int64_t b = cu_seqlens ? 0 : n;
        const int64_t bos = cu_seqlens ? cu_seqlens[n] : 0;
        const int64_t eos = cu_seqlens ? cu_seqlens[n + 1] : T;
        double* S = (double*)malloc(sizeof(double) * Dk * Dv);
        rows_t r = {0};
        if (!S || !rows_alloc(&r, Dk, Dv)) { free(S); rows_free(&r); failed |= 1; continue; }
        const int64_t s_off = (n * H + h) * Dk * Dv;
        for (int64_t e = 0; e < Dk * Dv; ++e)
            S[e] = initial_state ? (double)initial_state[s_off + e] : 0.0;
        for (int64_t t = bos; t < eos; ++t) {
            const int64_t row = (b * T + t) * H + h;
            widen(q + row * Dk, r.q, Dk);
            widen(k + row * Dk, r.k, Dk);
            widen(g + row * Dk, r.g, Dk);
            widen(v + row * Dv, r.v, Dv);
            kda_ref_token(S, r.x, r.q, r.k, r.v, r.g, (double)beta[row], Dk, Dv, scale, o + row * Dv);
        }
        if (final_state) memcpy(final_state + s_off, S, sizeof(double) * Dk * Dv);
        free(S);
        rows_free(&r);
    }
    return failed ? -1 : 0;
}

/*
 * One decode step: every row r (one token) updates state_cache[slot(r), h] in
 * place, where slot(r) = slots ? slots[r] : r. q,k,g [Nb,H,Dk]; v [Nb,H,Dv];
 * beta [Nb,H]; state_cache [n_slots,H,Dk,Dv] (double, updated); o [Nb,H,Dv].
 */
int kda_ref_decode_step(const float* q, const float* k, const float* v, const float* g,
                        const float* beta, double* state_cache, const int64_t* slots,
                        int64_t n_slots, int64_t Nb, int64_t H, int64_t Dk, int64_t Dv,
                        double scale, double* o, int nthreads)
{
    if (!q || !k || !v || !g || !beta || !state_cache || !o || Nb < 0 || H < 1 || Dk < 1 || Dv < 1)
        return -1;
    for (int64_t r = 0; r < Nb; ++r) {
        const int64_t s = slots ? slots[r] : r;
        if (s < 0 || s >= n_slots) return -1;
        for (int64_t r2 = 0; r2 < r; ++r2)   /* two rows may not share a slot */
            if ((slots ? slots[r2] : r2) == s) return -1;
    }
    int failed = 0;
    const int64_t units = Nb * H;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads) reduction(| : failed)
#endif
    for (int64_t u = 0; u < units; ++u) {
        const int64_t r = u / H, h = u % H;
        const int64_t s = slots ? slots[r] : r;
        rows_t w = {0};
        if (!rows_alloc(&w, Dk, Dv)) { rows_free(&w); failed |= 1; continue; }
        const int64_t row = r * H + h;
        widen(q + row * Dk, w.q, Dk);
        widen(k + row * Dk, w.k, Dk);
        widen(g + row * Dk, w.g, Dk);
        widen(v + row * Dv, w.v, Dv);
        kda_ref_token(state_cache + (s * H + h) * Dk * Dv, w.x, w.q, w.k, w.v, w.g, (double)beta[row],
                      Dk, Dv, scale, o + row * Dv);
        rows_free(&w);
    }
    return failed ? -1 : 0;
}

/*
 * The gate, beta and normalisation prologue of one token-head, in double.
 * It is the reading of the pages' gate parameters documented with the
 * library: A_log has one entry per key channel, shared by every head; dt_bias
 * one per (head, key channel); the gate is bounded below by lb:
 *   q = q_raw / sqrt(|q_raw|^2 + eps),   k likewise
 *   g[c] = lb * sigmoid(exp(A_log[c]) * (g_logit[c] + dt_bias[c]))
 *   beta = sigmoid(beta_logit)
 * Returns beta; writes q, k, g [Dk].
 */
static double kda_ref_prologue_token(const float* qr, const float* kr, const float* gl, double bl,
                                     const float* A_log, const float* dtb, double lb, double eps,
                                     int64_t Dk, double* q, double* k, double* g)
{
    double sq = 0.0, sk = 0.0;
    for (int64_t i = 0; i < Dk; ++i) {
        sq += (double)qr[i] * (double)qr[i];
        sk += (double)kr[i] * (double)kr[i];
    }
    const double nq = sqrt(sq + eps), nk = sqrt(sk + eps);
    for (int64_t i = 0; i < Dk; ++i) {
        q[i] = (double)qr[i] / nq;
        k[i] = (double)kr[i] / nk;
        const double z = exp((double)A_log[i]) * ((double)gl[i] + (double)dtb[i]);
        g[i] = lb / (1.0 + exp(-z));
    }
    return 1.0 / (1.0 + exp(-bl));
}

/*
 * Forward from the raw projections: q_raw, k_raw, g_logit [B,T,H,Dk], v
 * [B,T,H,Dv], beta_logit [B,T,H], A_log [Dk], dt_bias [H*Dk]; each token goes
 * through the prologue above, then the recurrence. Other arguments and the
 * return value as kda_ref_forward.
 */
int kda_ref_prologue_forward(const float* q_raw, const float* k_raw, const float* v,
                             const float* g_logit, const float* beta_logit,
                             const float* A_log, const float* dt_bias, double lb, double eps,
                             const float* initial_state, const int64_t* cu_seqlens, int64_t N,
                             int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                             double scale, double* o, double* final_state, int nthreads)
{
    if (!q_raw || !k_raw || !v || !g_logit || !beta_logit || !A_log || !dt_bias || !o ||
        B < 1 || T < 0 || H < 1 || Dk < 1 || Dv < 1 || !(eps >= 0.0))
        return -1;
    if (cu_seqlens) {
        if (B != 1 || N < 1 || cu_seqlens[0] != 0 || cu_seqlens[N] != T) return -1;
        for (int64_t n = 0; n < N; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    } else {
        N = B;
    }
    int failed = 0;
    const int64_t units = N * H;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : failed)
#endif
    for (int64_t u = 0; u < units; ++u) {
        const int64_t n = u / H, h = u % H;
        const int64_t b = cu_seqlens ? 0 : n;
        const int64_t bos = cu_seqlens ? cu_seqlens[n] : 0;
        const int64_t eos = cu_seqlens ? cu_seqlens[n + 1] : T;
        double* S = (double*)malloc(sizeof(double) * Dk * Dv);
        rows_t r = {0};
        if (!S || !rows_alloc(&r, Dk, Dv)) { free(S); rows_free(&r); failed |= 1; continue; }
        const int64_t s_off = (n * H + h) * Dk * Dv;
        for (int64_t e = 0; e < Dk * Dv; ++e)
            S[e] = initial_state ? (double)initial_state[s_off + e] : 0.0;
        for (int64_t t = bos; t < eos; ++t) {
            const int64_t row = (b * T + t) * H + h;
            const double bt = kda_ref_prologue_token(q_raw + row * Dk, k_raw + row * Dk, g_logit + row * Dk,
                                                     (double)beta_logit[row], A_log, dt_bias + h * Dk,
                                                     lb, eps, Dk, r.q, r.k, r.g);
            widen(v + row * Dv, r.v, Dv);
            kda_ref_token(S, r.x, r.q, r.k, r.v, r.g, bt, Dk, Dv, scale, o + row * Dv);
        }
        if (final_state) memcpy(final_state + s_off, S, sizeof(double) * Dk * Dv);
        free(S);
        rows_free(&r);
    }
    return failed ? -1 : 0;
}

/*
 * Short causal depthwise convolution over time (kernel 4), the step before the
 * KDA projections enter the recurrence (hysenlabs "kimi-k3-mlx", section
 * "Attention is 93 layers ...": a short convolution with kernel size 4 on the
 * query, key and value projections). Per sequence n and channel c, with the
 * window ending at token t:
 *   y[t][c] = sum_{i=0..3} w[c][i] * x[t - 3 + i][c]
 * where x before the sequence's first token comes from the conv state
 * (state[n][j][c] holds x[-3 + j]) or is 0 without one; then, with
 * activation = 1, y <- y * sigmoid(y). The final conv state holds the last
 * three inputs of the window (x[L-3 .. L-1], reaching into the initial state
 * when L < 3). x, y [B,T,C]; w [C][4]; states [N][3][C]. Returns 0, or -1 on
 * bad arguments.
 */
int kda_ref_short_conv(const float* x, const float* w, const float* state_in, const int64_t* cu_seqlens,
                       int64_t N, int64_t B, int64_t T, int64_t C, int activation, double* y,
                       double* state_out)
{
    if (!x || !w || !y || B < 1 || T < 0 || C < 1 || (activation != 0 && activation != 1)) return -1;
    if (cu_seqlens) {
        if (B != 1 || N < 1 || cu_seqlens[0] != 0 || cu_seqlens[N] != T) return -1;
        for (int64_t n = 0; n < N; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    } else {
        N = B;
    }
    for (int64_t n = 0; n < N; ++n) {
        const int64_t b = cu_seqlens ? 0 : n;
        const int64_t bos = cu_seqlens ? cu_seqlens[n] : 0;
        const int64_t L = (cu_seqlens ? cu_seqlens[n + 1] : T) - bos;
        for (int64_t c = 0; c < C; ++c) {
            /* the input sequence extended by the three state values in front */
            #define XIN(tau) ((tau) >= 0 ? (double)x[((b * T) + bos + (tau)) * C + c] \
                              : (state_in ? (double)state_in[(n * 3 + (3 + (tau))) * C + c] : 0.0))
            for (int64_t t = 0; t < L; ++t) {
                double acc = 0.0;
                for (int i = 0; i < 4; ++i) acc += (double)w[c * 4 + i] * XIN(t - 3 + i);
                if (activation) acc = acc / (1.0 + exp(-acc));
                y[((b * T) + bos + t) * C + c] = acc;
            }
            if (state_out)
                for (int j = 0; j < 3; ++j) state_out[(n * 3 + j) * C + c] = XIN(L - 3 + j);
            #undef XIN
        }
    }
    return 0;
}

/*
 * One decode step of the convolution: row r (one token) reads and updates
 * cache[slot(r)] ([3][C], the last three inputs), slot(r) = slots ? slots[r] : r.
 * x, y [Nb][C]; cache [n_slots][3][C] (double, updated in place).
 */
int kda_ref_short_conv_step(const float* x, const float* w, double* cache, const int64_t* slots,
                            int64_t n_slots, int64_t Nb, int64_t C, int activation, double* y)
{
    if (!x || !w || !cache || !y || Nb < 0 || C < 1 || (activation != 0 && activation != 1)) return -1;
    for (int64_t r = 0; r < Nb; ++r) {
        const int64_t s = slots ? slots[r] : r;
        if (s < 0 || s >= n_slots) return -1;
        double* st = cache + s * 3 * C;
        for (int64_t c = 0; c < C; ++c) {
            const double win[4] = {st[c], st[C + c], st[2 * C + c], (double)x[r * C + c]};
            double acc = 0.0;
            for (int i = 0; i < 4; ++i) acc += (double)w[c * 4 + i] * win[i];
            if (activation) acc = acc / (1.0 + exp(-acc));
            y[r * C + c] = acc;
            st[c] = win[1];
            st[C + c] = win[2];
            st[2 * C + c] = win[3];
        }
    }
    return 0;
}

/*
 * Reverse-mode gradient of the recurrence (the forward of kda_ref_forward)
 * for the loss  L = sum_t <d_o[t], o[t]> + <d_final, S_T>  per sequence and
 * head, written out step by step from the forward's definition:
 *   S' = Diag(e^g) S_{t-1};  x = S'^T k;  u = beta (v - x);  S_t = S' + k u^T;
 *   o = scale S_t^T q.
 * Going backward with dS (= dL/dS_t, starting from d_final or 0):
 *   dS += scale q do^T;           dq = scale S_t do
 *   du = dS^T k;  dk = dS u;      dbeta = du . (v - x);  dv = beta du
 *   dx = -beta du;  dk += S' dx;  dS' = dS + k dx^T
 *   dg = rowsum(dS' * S');        dS_{t-1} = Diag(e^g) dS'
 * The states S_{t-1} come from a forward recomputation: one checkpoint every
 * 64 tokens, the 64 states of a block re-run from it. Outputs (double):
 * dq, dk, dg [B,T,H,Dk], dv [B,T,H,Dv], dbeta [B,T,H], d_initial [N,H,Dk,Dv]
 * (may be NULL). Rows outside every sequence are left untouched. Returns 0,
 * or -1 on bad arguments / no memory.
 */
int kda_ref_backward(const float* q, const float* k, const float* v, const float* g, const float* beta,
                     const float* initial_state, const int64_t* cu_seqlens, const float* d_o,
                     const float* d_final, int64_t N, int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                     double scale, double* dq, double* dk, double* dv, double* dg, double* dbeta,
                     double* d_initial, int nthreads)
{
    if (!q || !k || !v || !g || !beta || !d_o || !dq || !dk || !dv || !dg || !dbeta || B < 1 || T < 0 ||
        H < 1 || Dk < 1 || Dv < 1)
        return -1;
    if (cu_seqlens) {
        if (B != 1 || N < 1 || cu_seqlens[0] != 0 || cu_seqlens[N] != T) return -1;
        for (int64_t n = 0; n < N; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    } else {
        N = B;
    }
    enum { BLK = 64 };
    int failed = 0;
    const int64_t units = N * H;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : failed)
#endif
    for (int64_t uidx = 0; uidx < units; ++uidx) {
        const int64_t n = uidx / H, h = uidx % H;
        const int64_t b = cu_seqlens ? 0 : n;
        const int64_t bos = cu_seqlens ? cu_seqlens[n] : 0;
        const int64_t eos = cu_seqlens ? cu_seqlens[n + 1] : T;
        const int64_t L = eos - bos, SZ = Dk * Dv;
        const int64_t nblk = (L + BLK - 1) / BLK;
        double* ckpt = (double*)malloc(sizeof(double) * SZ * (nblk > 0 ? nblk : 1));
        double* states = (double*)malloc(sizeof(double) * SZ * BLK);   /* S_{t-1} of one block */
        double* S = (double*)malloc(sizeof(double) * SZ);
        double* dS = (double*)malloc(sizeof(double) * SZ);
        double* Sd = (double*)malloc(sizeof(double) * SZ);
        double* vec = (double*)malloc(sizeof(double) * (4 * Dv + 2 * Dk));
        rows_t r = {0};
        if (!ckpt || !states || !S || !dS || !Sd || !vec || !rows_alloc(&r, Dk, Dv)) {
            free(ckpt); free(states); free(S); free(dS); free(Sd); free(vec); rows_free(&r);
            failed |= 1;
            continue;
        }
        double *x = vec, *u = vec + Dv, *du = vec + 2 * Dv, *dx = vec + 3 * Dv;
        const int64_t s_off = (n * H + h) * SZ;
        for (int64_t e = 0; e < SZ; ++e) S[e] = initial_state ? (double)initial_state[s_off + e] : 0.0;
        /* forward: checkpoint at the start of every block */
        for (int64_t t = 0; t < L; ++t) {
            if (t % BLK == 0) memcpy(ckpt + (t / BLK) * SZ, S, sizeof(double) * SZ);
            const int64_t row = (b * T + bos + t) * H + h;
            widen(q + row * Dk, r.q, Dk); widen(k + row * Dk, r.k, Dk);
            widen(g + row * Dk, r.g, Dk); widen(v + row * Dv, r.v, Dv);
            kda_ref_token(S, r.x, r.q, r.k, r.v, r.g, (double)beta[row], Dk, Dv, scale, NULL);
        }
        for (int64_t e = 0; e < SZ; ++e) dS[e] = d_final ? (double)d_final[s_off + e] : 0.0;
        for (int64_t blk = nblk - 1; blk >= 0; --blk) {
            const int64_t t0 = blk * BLK, t1 = (t0 + BLK < L) ? t0 + BLK : L;
            memcpy(S, ckpt + blk * SZ, sizeof(double) * SZ);
            for (int64_t t = t0; t < t1; ++t) {
                memcpy(states + (t - t0) * SZ, S, sizeof(double) * SZ);
                const int64_t row = (b * T + bos + t) * H + h;
                widen(q + row * Dk, r.q, Dk); widen(k + row * Dk, r.k, Dk);
                widen(g + row * Dk, r.g, Dk); widen(v + row * Dv, r.v, Dv);
                kda_ref_token(S, r.x, r.q, r.k, r.v, r.g, (double)beta[row], Dk, Dv, scale, NULL);
            }
            for (int64_t t = t1 - 1; t >= t0; --t) {
                const int64_t row = (b * T + bos + t) * H + h;
                widen(q + row * Dk, r.q, Dk); widen(k + row * Dk, r.k, Dk);
                widen(g + row * Dk, r.g, Dk); widen(v + row * Dv, r.v, Dv);
                const double bt = (double)beta[row];
                const double* Sp = states + (t - t0) * SZ;            /* S_{t-1} */
                const float* dot = d_o + row * Dv;
                /* S' = Diag(e^g) S_{t-1}; x = S'^T k; u = beta (v - x) */
                for (int64_t i = 0; i < Dk; ++i) {
                    const double a = exp(r.g[i]);
                    for (int64_t j = 0; j < Dv; ++j) Sd[i * Dv + j] = a * Sp[i * Dv + j];
                }
                for (int64_t j = 0; j < Dv; ++j) x[j] = 0.0;
                for (int64_t i = 0; i < Dk; ++i)
                    for (int64_t j = 0; j < Dv; ++j) x[j] += r.k[i] * Sd[i * Dv + j];
                for (int64_t j = 0; j < Dv; ++j) u[j] = bt * (r.v[j] - x[j]);
                /* o = scale (S' + k u^T)^T q */
                for (int64_t i = 0; i < Dk; ++i) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < Dv; ++j) {
                        dS[i * Dv + j] += scale * r.q[i] * (double)dot[j];
                        acc += (Sd[i * Dv + j] + r.k[i] * u[j]) * (double)dot[j];
                    }
                    dq[row * Dk + i] = scale * acc;
                }
                /* S_t = S' + k u^T */
                for (int64_t j = 0; j < Dv; ++j) du[j] = 0.0;
                for (int64_t i = 0; i < Dk; ++i) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < Dv; ++j) {
                        du[j] += dS[i * Dv + j] * r.k[i];
                        acc += dS[i * Dv + j] * u[j];
                    }
                    dk[row * Dk + i] = acc;
                }
                double dbt = 0.0;
                for (int64_t j = 0; j < Dv; ++j) {
                    dbt += du[j] * (r.v[j] - x[j]);
                    dv[row * Dv + j] = bt * du[j];
                    dx[j] = -bt * du[j];
                }
                dbeta[row] = dbt;
                /* x = S'^T k;  S' = Diag(e^g) S_{t-1} */
                for (int64_t i = 0; i < Dk; ++i) {
                    const double a = exp(r.g[i]);
                    double acc = 0.0, dgi = 0.0;
                    for (int64_t j = 0; j < Dv; ++j) {
                        acc += Sd[i * Dv + j] * dx[j];
                        const double dsd = dS[i * Dv + j] + r.k[i] * dx[j];
                        dgi += dsd * Sd[i * Dv + j];
                        dS[i * Dv + j] = a * dsd;
                    }
                    dk[row * Dk + i] += acc;
                    dg[row * Dk + i] = dgi;
                }
            }
        }
        if (d_initial) memcpy(d_initial + s_off, dS, sizeof(double) * SZ);
        free(ckpt); free(states); free(S); free(dS); free(Sd); free(vec); rows_free(&r);
    }
    return failed ? -1 : 0;
}
