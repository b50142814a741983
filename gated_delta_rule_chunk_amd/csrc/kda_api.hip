// C ABI of libkda.so: argument validation, kernel selection, error mapping.
// Every check runs on the host before any launch; a rejected call touches no
// memory and makes no HIP call.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "../../include/kda.h"
#include "launchers.hpp"

// Device status words, counted since the module was loaded on this device:
// [0] bounded waits between waves (in any kernel of this library) that gave
// up; [1] waves of the matrix-core forward or backward that met log-decays out
// of the range they need. Kernels add to them with a vector atomic from one lane; the host
// only reads them (kda_device_check). The rest of the array is padding.
__device__ __attribute__((aligned(256))) unsigned int kda_device_status[64];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_dev_mutex;
unsigned int* g_status_ptr[kMaxDevices] = {};
unsigned int g_status_seen[kMaxDevices][2] = {};   // [0] wait give-ups, [1] gates out of range
std::atomic<int> g_spin_limit{1 << 22};

}  // namespace

namespace kda {

// The status word's device address on the current device, looked up once per
// device (each device holds its own copy of the module's variables).
unsigned int* device_status_word() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_dev_mutex);
    if (!g_status_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(kda_device_status)) != hipSuccess) return nullptr;
        g_status_ptr[dev] = static_cast<unsigned int*>(p);
    }
    return g_status_ptr[dev];
}

int wait_spin_limit() { return g_spin_limit.load(std::memory_order_relaxed); }

}  // namespace kda

namespace {

thread_local char g_last_error[512] = "";

kda_status fail(kda_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

bool dim_ok(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

constexpr int32_t KDA_MAX_SEGMENTS = 4096;

}  // namespace

extern "C" {

const char* kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
        case KDA_ERR_HIP: return "KDA_ERR_HIP";
        case KDA_ERR_DEVICE: return "KDA_ERR_DEVICE";
    }
    return "KDA_UNKNOWN_STATUS";
}

const char* kda_last_error_message(void) { return g_last_error; }

kda_status kda_set_wait_limit(int32_t polls) {
    g_last_error[0] = 0;
    if (polls < 0) return fail(KDA_ERR_INVALID_ARG, "kda_set_wait_limit: polls must be >= 0, got %d", polls);
    g_spin_limit.store(polls, std::memory_order_relaxed);
    return KDA_OK;
}

kda_status kda_device_check(void* stream) {
    g_last_error[0] = 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    unsigned int* word = kda::device_status_word();
    int dev = 0;
    if (!word || hipGetDevice(&dev) != hipSuccess)
        return fail(KDA_ERR_HIP, "kda_device_check: the device status word is not accessible");
    unsigned int now[2] = {0, 0};
    hipError_t e = hipMemcpyAsync(now, word, sizeof(now), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "kda_device_check: %s", hipGetErrorString(e));
    unsigned int seen[2];
    {
        std::lock_guard<std::mutex> lock(g_dev_mutex);
        seen[0] = g_status_seen[dev][0];
        seen[1] = g_status_seen[dev][1];
        g_status_seen[dev][0] = now[0];
        g_status_seen[dev][1] = now[1];
    }
    if (now[0] != seen[0])
        return fail(KDA_ERR_DEVICE,
                    "kda_device_check: %u bounded wait(s) between waves gave up on device %d since the last check; "
                    "the outputs of the calls that ran meanwhile are not valid",
                    now[0] - seen[0], dev);
    if (now[1] != seen[1])
        return fail(KDA_ERR_DEVICE,
                    "kda_device_check: a matrix-core kernel met log-decays g out of its range (forward: a 16-row "
                    "chunk's total outside [-84, 0]; backward: a g outside [-5, 0]; NaN included) in %u wave(s) on "
                    "device %d since the last check; the outputs of the calls that ran meanwhile are not valid",
                    now[1] - seen[1], dev);
    return KDA_OK;
}

}  // extern "C"

namespace {

// Checks shared by the two chunk entry points; fills a on success.
kda_status check_chunk(const char* fn, const void* q, const void* k, const void* v, const void* g,
                       const void* beta, const float* initial_state, const int32_t* cu_seqlens,
                       int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t N,
                       int32_t chunk_size, float scale, kda_dtype dtype, void* o, float* final_state,
                       kda::ChunkArgs& a) {
    if (T > 0 && (!q || !k || !v || !g || !beta || !o))
        return fail(KDA_ERR_INVALID_ARG, "%s: every input and o must be non-NULL when T > 0", fn);
    if (B < 1 || T < 0 || H < 1 || N < 0)
        return fail(KDA_ERR_INVALID_ARG, "%s: need B >= 1, T >= 0, H >= 1, N >= 0 (got B=%d T=%d H=%d N=%d)",
                    fn, B, T, H, N);
    if (dtype != KDA_F32 && dtype != KDA_BF16)
        return fail(KDA_ERR_UNSUPPORTED, "%s: dtype %d is not KDA_F32 or KDA_BF16", fn, (int)dtype);
    if (!dim_ok(Dk) || !dim_ok(Dv))
        return fail(KDA_ERR_UNSUPPORTED, "%s: Dk=%d, Dv=%d; supported head dims are 16, 32, 64, 128",
                    fn, Dk, Dv);
    const int32_t chunk = chunk_size == 0 ? 16 : chunk_size;
    if (chunk != 16 && chunk != 32 && chunk != 64)
        return fail(KDA_ERR_UNSUPPORTED, "%s: chunk_size=%d; supported are 16, 32, 64 (0 = 16)", fn, chunk_size);
    if (cu_seqlens) {
        if (B != 1)
            return fail(KDA_ERR_INVALID_ARG, "%s: packed sequences (cu_seqlens) need B == 1, got B=%d", fn, B);
        if (N < 1)
            return fail(KDA_ERR_INVALID_ARG, "%s: packed sequences need N >= 1, got N=%d", fn, N);
    } else if (N != B) {
        return fail(KDA_ERR_INVALID_ARG, "%s: without cu_seqlens N must equal B (N=%d, B=%d)", fn, N, B);
    }
    const int64_t units = (int64_t)N * H;
    if (units > (int64_t)1 << 26 || (int64_t)B * T * H > ((int64_t)1 << 40))
        return fail(KDA_ERR_UNSUPPORTED, "%s: problem too large (N*H=%lld)", fn, (long long)units);
    if (T > 0 && (o == q || o == k || o == v || o == g || o == beta))
        return fail(KDA_ERR_INVALID_ARG, "%s: o must not alias an input", fn);
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.s0 = initial_state; a.cu = cu_seqlens; a.o = o; a.sT = final_state;
    a.B = B; a.T = T; a.H = H; a.Dk = Dk; a.Dv = Dv; a.N = N; a.chunk = chunk; a.chunk_req = chunk_size;
    a.scale = scale; a.bf16 = dtype == KDA_BF16;
    return KDA_OK;
}

// The matrix-core kernel has one chunk length (16 rows); an explicit request
// for another one is refused rather than ignored.
kda_status check_kernel_chunk(const char* fn, const kda::ChunkArgs& a) {
    if (kda::chunk_mfma_supported(a) && a.chunk_req != 0 && a.chunk_req != 16)
        return fail(KDA_ERR_UNSUPPORTED,
                    "%s: chunk_size=%d; the bf16 Dk = Dv = 128 kernel runs 16-row chunks (pass 0 or 16)", fn,
                    a.chunk_req);
    return KDA_OK;
}

// Points a's bounded waits at the current device's status word.
kda_status attach_status(const char* fn, kda::ChunkArgs& a) {
    a.status = kda::device_status_word();
    a.spin_limit = kda::wait_spin_limit();
    if (!a.status) return fail(KDA_ERR_HIP, "%s: the device status word is not accessible", fn);
    return KDA_OK;
}

kda_status launch_chunk(const char* fn, kda::ChunkArgs a, void* stream) {
    const kda_status cs = check_kernel_chunk(fn, a);
    if (cs != KDA_OK) return cs;
    if ((int64_t)a.N * a.H == 0) return KDA_OK;
    const kda_status ss = attach_status(fn, a);
    if (ss != KDA_OK) return ss;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = kda::chunk_mfma_supported(a) ? kda::launch_chunk_mfma(a, s)
                                                      : kda::launch_chunk_generic(a, s);
    if (e != hipSuccess)
        return fail(KDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return KDA_OK;
}

}  // namespace

namespace {

// Checks shared by the decode entry points; fills a on success.
kda_status check_step(const char* fn, const void* q, const void* k, const void* v, const void* g, const void* beta,
                      float* state_cache, const int32_t* state_slots, int32_t n_slots, int32_t Nb, int32_t H,
                      int32_t Dk, int32_t Dv, float scale, kda_dtype dtype, void* o, kda::StepArgs& a) {
    if (Nb != 0 && (!q || !k || !v || !g || !beta || !state_cache || !o))
        return fail(KDA_ERR_INVALID_ARG, "%s: q, k, v, g, beta, state_cache and o must be non-NULL", fn);
    if (Nb < 0 || H < 1 || n_slots < 0)
        return fail(KDA_ERR_INVALID_ARG, "%s: need Nb >= 0, H >= 1, n_slots >= 0 (got %d, %d, %d)", fn, Nb, H,
                    n_slots);
    if (dtype != KDA_F32 && dtype != KDA_BF16)
        return fail(KDA_ERR_UNSUPPORTED, "%s: dtype %d is not KDA_F32 or KDA_BF16", fn, (int)dtype);
    if (!dim_ok(Dk) || !dim_ok(Dv))
        return fail(KDA_ERR_UNSUPPORTED, "%s: Dk=%d, Dv=%d; supported head dims are 16, 32, 64, 128", fn, Dk, Dv);
    if (!state_slots && Nb > n_slots)
        return fail(KDA_ERR_INVALID_ARG,
                    "%s: without state_slots row r uses slot r, so Nb (%d) must be <= n_slots (%d)", fn, Nb,
                    n_slots);
    if ((int64_t)Nb * H > ((int64_t)1 << 30)) return fail(KDA_ERR_UNSUPPORTED, "%s: Nb*H too large", fn);
    if (Nb != 0 && (o == q || o == k || o == v || o == g || o == beta || o == state_cache))
        return fail(KDA_ERR_INVALID_ARG, "%s: o must not alias an input", fn);
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.cache = state_cache; a.slots = state_slots; a.o = o;
    a.n_slots = n_slots; a.Nb = Nb; a.H = H; a.Dk = Dk; a.Dv = Dv; a.scale = scale; a.bf16 = dtype == KDA_BF16;
    return KDA_OK;
}

// The prologue's parameters of a decode entry point.
kda_status check_step_prologue(const char* fn, const float* A_log, const float* dt_bias, float gate_lower_bound,
                               float l2_eps, int32_t Nb, kda::StepArgs& a) {
    if (Nb != 0 && (!A_log || !dt_bias))
        return fail(KDA_ERR_INVALID_ARG, "%s: A_log and dt_bias must be non-NULL when Nb > 0", fn);
    if (!(gate_lower_bound < 0.f) || !(gate_lower_bound > -1e30f))
        return fail(KDA_ERR_INVALID_ARG, "%s: gate_lower_bound must be finite and negative (got %g)", fn,
                    (double)gate_lower_bound);
    if (!(l2_eps > 0.f) || !(l2_eps < 1e30f))
        return fail(KDA_ERR_INVALID_ARG, "%s: l2_eps must be finite and positive (got %g)", fn, (double)l2_eps);
    a.prologue = true;
    a.A_log = A_log;
    a.dt_bias = dt_bias;
    a.gate_lb = gate_lower_bound;
    a.l2_eps = l2_eps;
    return KDA_OK;
}

kda_status launch_step(const char* fn, const kda::StepArgs& a, void* stream) {
    const hipError_t e = kda::launch_recurrent_step(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const float* initial_state,
                         const int32_t* cu_seqlens, int32_t B, int32_t T, int32_t H,
                         int32_t Dk, int32_t Dv, int32_t N, int32_t chunk_size, float scale,
                         kda_dtype dtype, void* o, float* final_state, void* stream) {
    g_last_error[0] = 0;
    kda::ChunkArgs a;
    const kda_status st = check_chunk("kda_chunk_fwd", q, k, v, g, beta, initial_state, cu_seqlens, B, T, H,
                                      Dk, Dv, N, chunk_size, scale, dtype, o, final_state, a);
    if (st != KDA_OK) return st;
    return launch_chunk("kda_chunk_fwd", a, stream);
}

kda_status kda_chunk_fwd_prologue(const void* q_raw, const void* k_raw, const void* v,
                                  const void* g_logit, const void* beta_logit, const float* A_log,
                                  const float* dt_bias, float gate_lower_bound, float l2_eps,
                                  const float* initial_state, const int32_t* cu_seqlens, int32_t B,
                                  int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t N,
                                  int32_t chunk_size, float scale, kda_dtype dtype, void* o,
                                  float* final_state, void* stream) {
    g_last_error[0] = 0;
    const char* fn = "kda_chunk_fwd_prologue";
    kda::ChunkArgs a;
    const kda_status st = check_chunk(fn, q_raw, k_raw, v, g_logit, beta_logit, initial_state, cu_seqlens, B,
                                      T, H, Dk, Dv, N, chunk_size, scale, dtype, o, final_state, a);
    if (st != KDA_OK) return st;
    if (T > 0 && (!A_log || !dt_bias))
        return fail(KDA_ERR_INVALID_ARG, "%s: A_log and dt_bias must be non-NULL when T > 0", fn);
    if (!(gate_lower_bound < 0.f) || !(gate_lower_bound > -1e30f))
        return fail(KDA_ERR_INVALID_ARG, "%s: gate_lower_bound must be finite and negative (got %g)", fn,
                    (double)gate_lower_bound);
    if (!(l2_eps > 0.f) || !(l2_eps < 1e30f))
        return fail(KDA_ERR_INVALID_ARG, "%s: l2_eps must be finite and positive (got %g)", fn, (double)l2_eps);
    a.prologue = true;
    a.A_log = A_log;
    a.dt_bias = dt_bias;
    a.gate_lb = gate_lower_bound;
    a.l2_eps = l2_eps;
    return launch_chunk(fn, a, stream);
}

size_t kda_chunk_fwd_conv_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, kda_dtype dtype,
                                          float gate_lower_bound) {
    if (B < 1 || T <= 0 || H < 1 || !dim_ok(Dk) || !dim_ok(Dv) || (dtype != KDA_F32 && dtype != KDA_BF16)) return 0;
    const int64_t rows = (int64_t)B * T * H;
    const bool fused = dtype == KDA_BF16 && Dk == 128 && Dv == 128 && gate_lower_bound >= -5.f;
    // fused: the convolved q and k (bf16); otherwise the three convolved projections
    return fused ? (size_t)(2 * rows * Dk * 2) : (size_t)(rows * (2 * Dk + Dv) * (dtype == KDA_BF16 ? 2 : 4));
}

kda_status kda_chunk_fwd_conv(const void* xq, const void* xk, const void* xv, const float* wq, const float* wk,
                              const float* wv, const float* conv_state_q, const float* conv_state_k,
                              const float* conv_state_v, int32_t activation, const void* g_logit,
                              const void* beta_logit, const float* A_log, const float* dt_bias,
                              float gate_lower_bound, float l2_eps, const float* initial_state,
                              const int32_t* cu_seqlens, int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv,
                              int32_t N, int32_t chunk_size, float scale, kda_dtype dtype, void* workspace,
                              size_t workspace_bytes, void* o, float* final_state, float* conv_state_q_out,
                              float* conv_state_k_out, float* conv_state_v_out, void* stream) {
    g_last_error[0] = 0;
    const char* fn = "kda_chunk_fwd_conv";
    kda::ChunkArgs a;
    const kda_status st = check_chunk(fn, xq, xk, xv, g_logit, beta_logit, initial_state, cu_seqlens, B, T, H, Dk,
                                      Dv, N, chunk_size, scale, dtype, o, final_state, a);
    if (st != KDA_OK) return st;
    if (T > 0 && (!A_log || !dt_bias))
        return fail(KDA_ERR_INVALID_ARG, "%s: A_log and dt_bias must be non-NULL when T > 0", fn);
    if (!wq || !wk || !wv) return fail(KDA_ERR_INVALID_ARG, "%s: the conv taps wq, wk, wv must be non-NULL", fn);
    if (activation != 0 && activation != 1)
        return fail(KDA_ERR_INVALID_ARG, "%s: activation must be 0 (none) or 1 (SiLU), got %d", fn, activation);
    if (!(gate_lower_bound < 0.f) || !(gate_lower_bound > -1e30f))
        return fail(KDA_ERR_INVALID_ARG, "%s: gate_lower_bound must be finite and negative (got %g)", fn,
                    (double)gate_lower_bound);
    if (!(l2_eps > 0.f) || !(l2_eps < 1e30f))
        return fail(KDA_ERR_INVALID_ARG, "%s: l2_eps must be finite and positive (got %g)", fn, (double)l2_eps);
    if ((int64_t)B * T > ((int64_t)1 << 31) * 16)
        return fail(KDA_ERR_UNSUPPORTED, "%s: problem too large", fn);
    a.prologue = true;
    a.A_log = A_log;
    a.dt_bias = dt_bias;
    a.gate_lb = gate_lower_bound;
    a.l2_eps = l2_eps;
    const kda_status cs = check_kernel_chunk(fn, a);
    if (cs != KDA_OK) return cs;
    const size_t need = kda_chunk_fwd_conv_workspace_bytes(B, T, H, Dk, Dv, dtype, gate_lower_bound);
    if (workspace_bytes < need || (need > 0 && !workspace))
        return fail(KDA_ERR_INVALID_ARG, "%s: workspace of %zu bytes needed, got %zu%s", fn, need, workspace_bytes,
                    workspace ? "" : " (NULL)");
    if (need > 0) {
        const char* ws = static_cast<const char*>(workspace);
        const void* ptrs[] = {xq, xk, xv, g_logit, beta_logit, o, initial_state, final_state, wq, wk, wv,
                              conv_state_q, conv_state_k, conv_state_v, conv_state_q_out, conv_state_k_out,
                              conv_state_v_out};
        for (const void* p : ptrs) {
            const char* c = static_cast<const char*>(p);
            if (c && c >= ws && c < ws + need)
                return fail(KDA_ERR_INVALID_ARG, "%s: the workspace must not overlap an input or output", fn);
        }
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t rows = (int64_t)B * T * H;
    const bool fused = kda::chunk_mfma_supported(a);
    char* ws = static_cast<char*>(workspace);
    kda::ConvArgs c[3];
    const void* xs[3] = {xq, xk, xv};
    const float* wts[3] = {wq, wk, wv};
    const float* s0s[3] = {conv_state_q, conv_state_k, conv_state_v};
    float* s1s[3] = {conv_state_q_out, conv_state_k_out, conv_state_v_out};
    const int64_t elt = dtype == KDA_BF16 ? 2 : 4;
    for (int t = 0; t < 3; ++t) {
        c[t].x = xs[t]; c[t].w = wts[t]; c[t].state_in = s0s[t]; c[t].cu = cu_seqlens;
        c[t].y = fused ? nullptr : ws + (t == 0 ? 0 : t == 1 ? rows * Dk * elt : 2 * rows * Dk * elt);
        c[t].state_out = s1s[t];
        c[t].B = B; c[t].T = T; c[t].C = H * (t < 2 ? Dk : Dv); c[t].N = N;
        c[t].act = activation == 1; c[t].bf16 = dtype == KDA_BF16;
    }
    hipError_t e = hipSuccess;
    if (fused) {
        // q and k by the streaming convolution into the workspace (one
        // launch); v is convolved inside the chunk kernel by its state waves
        if (T > 0) {
            kda::ConvArgs ct[2] = {c[0], c[1]};
            for (int t = 0; t < 2; ++t) {
                ct[t].y = ws + t * rows * Dk * 2;
                ct[t].state_out = nullptr;
            }
            e = kda::launch_short_conv_set(ct, 2, s);
        }
        a.q = T > 0 ? ws : nullptr;
        a.k = T > 0 ? ws + rows * Dk * 2 : nullptr;
        a.v = xv;
        a.conv = true;
        a.conv_wv = wv;
        a.conv_sv = conv_state_v;
        a.conv_act = activation == 1;
        if (e == hipSuccess && (int64_t)a.N * a.H > 0) {
            const kda_status ss = attach_status(fn, a);
            if (ss != KDA_OK) return ss;
            e = kda::launch_chunk_mfma(a, s);
        }
    } else {
        // every other shape: the three convolutions into the workspace (one
        // launch), then the prologue forward
        if (T > 0) {
            kda::ConvArgs ct[3] = {c[0], c[1], c[2]};
            for (int t = 0; t < 3; ++t) ct[t].state_out = nullptr;
            e = kda::launch_short_conv_set(ct, 3, s);
        }
        if (e == hipSuccess) {
            a.q = c[0].y;
            a.k = c[1].y;
            a.v = c[2].y;
            if (T == 0) a.q = a.k = a.v = nullptr;
            const kda_status ls = launch_chunk(fn, a, stream);
            if (ls != KDA_OK) return ls;
        }
    }
    // final conv states (the last three inputs of every window), after
    // everything that reads the initial ones, which they may alias; one launch
    if (e == hipSuccess && N > 0 && (s1s[0] || s1s[1] || s1s[2])) {
        kda::ConvArgs ct[3] = {c[0], c[1], c[2]};
        for (int t = 0; t < 3; ++t) ct[t].y = nullptr;
        e = kda::launch_short_conv_set(ct, 3, s);
    }
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return KDA_OK;
}

size_t kda_chunk_fwd_split_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t N,
                                           kda_dtype dtype, int32_t segments) {
    if (B < 1 || T <= 0 || H < 1 || N < 1 || segments <= 1 || segments > KDA_MAX_SEGMENTS || !dim_ok(Dk) ||
        !dim_ok(Dv) || (dtype != KDA_F32 && dtype != KDA_BF16))
        return 0;
    kda::ChunkArgs a;
    a.B = B; a.T = T; a.H = H; a.Dk = Dk; a.Dv = Dv; a.N = N; a.bf16 = dtype == KDA_BF16;
    return (size_t)kda::split_layout(a, segments).bytes;
}

}  // extern "C"

namespace {

// The split's checks after the inputs', and its launch (shared by the plain
// and the raw-projection entry points).
kda_status run_split(const char* fn, kda::ChunkArgs& a, int32_t segments, void* workspace, size_t workspace_bytes,
                     void* stream) {
    const int32_t B = a.B, T = a.T, H = a.H, N = a.N;
    if (segments < 1 || segments > KDA_MAX_SEGMENTS)
        return fail(KDA_ERR_INVALID_ARG, "%s: segments must be in [1, %d], got %d", fn, KDA_MAX_SEGMENTS, segments);
    if ((int64_t)B * T > INT32_MAX || (int64_t)N * segments * H > ((int64_t)1 << 26))
        return fail(KDA_ERR_UNSUPPORTED, "%s: B*T must fit in int32 and N*segments*H below 2^26", fn);
    if (segments == 1 || T == 0) return launch_chunk(fn, a, stream);
    const kda_status cs = check_kernel_chunk(fn, a);
    if (cs != KDA_OK) return cs;
    const size_t need = kda_chunk_fwd_split_workspace_bytes(B, T, H, a.Dk, a.Dv, N, a.bf16 ? KDA_BF16 : KDA_F32,
                                                            segments);
    if (workspace_bytes < need || !workspace)
        return fail(KDA_ERR_INVALID_ARG, "%s: workspace of %zu bytes needed, got %zu%s", fn, need, workspace_bytes,
                    workspace ? "" : " (NULL)");
    {
        const char* ws = static_cast<const char*>(workspace);
        const void* ptrs[] = {a.q, a.k, a.v, a.g, a.beta, a.o, a.s0, a.sT, a.A_log, a.dt_bias};
        for (const void* p : ptrs) {
            const char* c = static_cast<const char*>(p);
            if (c && c >= ws && c < ws + need)
                return fail(KDA_ERR_INVALID_ARG, "%s: the workspace must not overlap an input or output", fn);
        }
    }
    const kda_status ss = attach_status(fn, a);
    if (ss != KDA_OK) return ss;
    const hipError_t e = kda::launch_chunk_fwd_split(a, segments, workspace, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_chunk_fwd_split(const void* q, const void* k, const void* v, const void* g, const void* beta,
                               const float* initial_state, const int32_t* cu_seqlens, int32_t B, int32_t T,
                               int32_t H, int32_t Dk, int32_t Dv, int32_t N, int32_t chunk_size, float scale,
                               kda_dtype dtype, int32_t segments, void* workspace, size_t workspace_bytes, void* o,
                               float* final_state, void* stream) {
    g_last_error[0] = 0;
    const char* fn = "kda_chunk_fwd_split";
    kda::ChunkArgs a;
    const kda_status st = check_chunk(fn, q, k, v, g, beta, initial_state, cu_seqlens, B, T, H, Dk, Dv, N,
                                      chunk_size, scale, dtype, o, final_state, a);
    if (st != KDA_OK) return st;
    return run_split(fn, a, segments, workspace, workspace_bytes, stream);
}

kda_status kda_chunk_fwd_split_prologue(const void* q_raw, const void* k_raw, const void* v, const void* g_logit,
                                        const void* beta_logit, const float* A_log, const float* dt_bias,
                                        float gate_lower_bound, float l2_eps, const float* initial_state,
                                        const int32_t* cu_seqlens, int32_t B, int32_t T, int32_t H, int32_t Dk,
                                        int32_t Dv, int32_t N, int32_t chunk_size, float scale, kda_dtype dtype,
                                        int32_t segments, void* workspace, size_t workspace_bytes, void* o,
                                        float* final_state, void* stream) {
    g_last_error[0] = 0;
    const char* fn = "kda_chunk_fwd_split_prologue";
    kda::ChunkArgs a;
    const kda_status st = check_chunk(fn, q_raw, k_raw, v, g_logit, beta_logit, initial_state, cu_seqlens, B, T, H,
                                      Dk, Dv, N, chunk_size, scale, dtype, o, final_state, a);
    if (st != KDA_OK) return st;
    if (T > 0 && (!A_log || !dt_bias))
        return fail(KDA_ERR_INVALID_ARG, "%s: A_log and dt_bias must be non-NULL when T > 0", fn);
    if (!(gate_lower_bound < 0.f) || !(gate_lower_bound > -1e30f))
        return fail(KDA_ERR_INVALID_ARG, "%s: gate_lower_bound must be finite and negative (got %g)", fn,
                    (double)gate_lower_bound);
    if (!(l2_eps > 0.f) || !(l2_eps < 1e30f))
        return fail(KDA_ERR_INVALID_ARG, "%s: l2_eps must be finite and positive (got %g)", fn, (double)l2_eps);
    a.prologue = true;
    a.A_log = A_log;
    a.dt_bias = dt_bias;
    a.gate_lb = gate_lower_bound;
    a.l2_eps = l2_eps;
    return run_split(fn, a, segments, workspace, workspace_bytes, stream);
}

kda_status kda_chunk_fwd_split_static(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                      const float* initial_state, const int32_t* cu_seqlens, int32_t B, int32_t T,
                                      int32_t H, int32_t Dk, int32_t Dv, int32_t N, int32_t chunk_size, float scale,
                                      kda_dtype dtype, int32_t segments, void* o, float* final_state, void* stream) {
    g_last_error[0] = 0;
    const char* fn = "kda_chunk_fwd_split_static";
    static_assert(KDA_SPLIT_STATIC_SCRATCH_BYTES == kda::kSplitStaticScratchBytes, "scratch size");
    kda::ChunkArgs a;
    const kda_status st = check_chunk(fn, q, k, v, g, beta, initial_state, cu_seqlens, B, T, H, Dk, Dv, N,
                                      chunk_size, scale, dtype, o, final_state, a);
    if (st != KDA_OK) return st;
    if (segments < 1 || segments > KDA_MAX_SEGMENTS)
        return fail(KDA_ERR_INVALID_ARG, "%s: segments must be in [1, %d], got %d", fn, KDA_MAX_SEGMENTS, segments);
    if ((int64_t)B * T > INT32_MAX || (int64_t)N * segments * H > ((int64_t)1 << 26))
        return fail(KDA_ERR_UNSUPPORTED, "%s: B*T must fit in int32 and N*segments*H below 2^26", fn);
    if (segments == 1 || T == 0) return launch_chunk(fn, a, stream);
    const kda_status cs = check_kernel_chunk(fn, a);
    if (cs != KDA_OK) return cs;
    const size_t need = kda_chunk_fwd_split_workspace_bytes(B, T, H, Dk, Dv, N, dtype, segments);
    if (need > kda::kSplitStaticScratchBytes)
        return fail(KDA_ERR_UNSUPPORTED,
                    "%s: these sizes need %zu bytes of scratch; the static scratch holds %zu "
                    "(use kda_chunk_fwd_split with a workspace)",
                    fn, need, (size_t)kda::kSplitStaticScratchBytes);
    void* ws = kda::split_static_scratch();
    if (!ws) return fail(KDA_ERR_HIP, "%s: the static scratch's device address could not be looked up", fn);
    const kda_status ss = attach_status(fn, a);
    if (ss != KDA_OK) return ss;
    const hipError_t e = kda::launch_chunk_fwd_split(a, segments, ws, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return KDA_OK;
}

size_t kda_chunk_bwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t N,
                                     int32_t packed) {
    if (B < 1 || T <= 0 || H < 1 || Dk < 1 || Dv < 1 || N < 0) return 0;
    return (size_t)kda::chunk_bwd_ws_floats(B, T, H, Dk, Dv, N, packed != 0) * sizeof(float);
}

kda_status kda_chunk_bwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                         const float* initial_state, const int32_t* cu_seqlens, const void* d_o,
                         const float* d_final_state, int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv,
                         int32_t N, float scale, kda_dtype dtype, void* workspace, size_t workspace_bytes,
                         float* dq, float* dk, float* dv, float* dg, float* dbeta, float* d_initial_state,
                         void* stream) {
    g_last_error[0] = 0;
    const char* fn = "kda_chunk_bwd";
    if (T > 0 && (!q || !k || !v || !g || !beta || !d_o))
        return fail(KDA_ERR_INVALID_ARG, "%s: q, k, v, g, beta and d_o must be non-NULL when T > 0", fn);
    if (T > 0 && (!dq || !dk || !dv || !dg || !dbeta))
        return fail(KDA_ERR_INVALID_ARG, "%s: dq, dk, dv, dg and dbeta must be non-NULL when T > 0", fn);
    if (B < 1 || T < 0 || H < 1 || N < 0)
        return fail(KDA_ERR_INVALID_ARG, "%s: need B >= 1, T >= 0, H >= 1, N >= 0 (got B=%d T=%d H=%d N=%d)",
                    fn, B, T, H, N);
    if (dtype != KDA_F32 && dtype != KDA_BF16)
        return fail(KDA_ERR_UNSUPPORTED, "%s: dtype %d is not KDA_F32 or KDA_BF16", fn, (int)dtype);
    if (!dim_ok(Dk) || !dim_ok(Dv))
        return fail(KDA_ERR_UNSUPPORTED, "%s: Dk=%d, Dv=%d; supported head dims are 16, 32, 64, 128", fn, Dk, Dv);
    if (cu_seqlens) {
        if (B != 1)
            return fail(KDA_ERR_INVALID_ARG, "%s: packed sequences (cu_seqlens) need B == 1, got B=%d", fn, B);
        if (N < 1) return fail(KDA_ERR_INVALID_ARG, "%s: packed sequences need N >= 1, got N=%d", fn, N);
    } else if (N != B) {
        return fail(KDA_ERR_INVALID_ARG, "%s: without cu_seqlens N must equal B (N=%d, B=%d)", fn, N, B);
    }
    if ((int64_t)N * H > ((int64_t)1 << 26) || (int64_t)B * T * H > ((int64_t)1 << 40))
        return fail(KDA_ERR_UNSUPPORTED, "%s: problem too large", fn);
    const size_t need = kda_chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, N, cu_seqlens != nullptr);
    if (workspace_bytes < need || (need > 0 && !workspace))
        return fail(KDA_ERR_INVALID_ARG, "%s: workspace of %zu bytes needed, got %zu%s", fn, need, workspace_bytes,
                    workspace ? "" : " (NULL)");
    if (T > 0) {
        const void* ins[] = {q, k, v, g, beta, d_o, workspace};
        const void* outs[] = {dq, dk, dv, dg, dbeta};
        for (const void* o : outs)
            for (const void* i : ins)
                if (o == i) return fail(KDA_ERR_INVALID_ARG, "%s: gradients must not alias an input", fn);
    }
    kda::BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.d_o = d_o;
    a.s0 = initial_state; a.cu = cu_seqlens; a.d_final = d_final_state;
    a.ws = static_cast<float*>(workspace);
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.d_s0 = d_initial_state;
    a.B = B; a.T = T; a.H = H; a.Dk = Dk; a.Dv = Dv; a.N = N; a.scale = scale; a.bf16 = dtype == KDA_BF16;
    if ((int64_t)N * H == 0) return KDA_OK;
    a.status = kda::device_status_word();
    if (!a.status) return fail(KDA_ERR_HIP, "%s: the device status word is not accessible", fn);
    const hipError_t e = kda::launch_chunk_bwd(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return KDA_OK;
}

size_t kda_chunk_bwd_prologue_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t N,
                                              int32_t packed) {
    if (B < 1 || T <= 0 || H < 1 || Dk < 1 || Dv < 1 || N < 0) return 0;
    return (size_t)kda::prologue_bwd_layout(B, T, H, Dk, Dv, N, packed != 0).bytes;
}

kda_status kda_chunk_bwd_prologue(const void* q_raw, const void* k_raw, const void* v, const void* g_logit,
                                  const void* beta_logit, const float* A_log, const float* dt_bias,
                                  float gate_lower_bound, float l2_eps, const float* initial_state,
                                  const int32_t* cu_seqlens, const void* d_o, const float* d_final_state, int32_t B,
                                  int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t N, float scale,
                                  kda_dtype dtype, void* workspace, size_t workspace_bytes, float* dq_raw,
                                  float* dk_raw, float* dv, float* dg_logit, float* dbeta_logit, float* dA_log,
                                  float* ddt_bias, float* d_initial_state, void* stream) {
    g_last_error[0] = 0;
    const char* fn = "kda_chunk_bwd_prologue";
    if (!A_log || !dt_bias || !dA_log || !ddt_bias)
        return fail(KDA_ERR_INVALID_ARG, "%s: A_log, dt_bias, dA_log and ddt_bias must be non-NULL", fn);
    if (!(gate_lower_bound < 0.f) || !(gate_lower_bound > -1e30f))
        return fail(KDA_ERR_INVALID_ARG, "%s: gate_lower_bound must be finite and negative (got %g)", fn,
                    (double)gate_lower_bound);
    if (!(l2_eps > 0.f) || !(l2_eps < 1e30f))
        return fail(KDA_ERR_INVALID_ARG, "%s: l2_eps must be finite and positive (got %g)", fn, (double)l2_eps);
    if (B < 1 || T < 0 || H < 1 || N < 0)
        return fail(KDA_ERR_INVALID_ARG, "%s: need B >= 1, T >= 0, H >= 1, N >= 0 (got B=%d T=%d H=%d N=%d)",
                    fn, B, T, H, N);
    if (dtype != KDA_F32 && dtype != KDA_BF16)
        return fail(KDA_ERR_UNSUPPORTED, "%s: dtype %d is not KDA_F32 or KDA_BF16", fn, (int)dtype);
    if (!dim_ok(Dk) || !dim_ok(Dv))
        return fail(KDA_ERR_UNSUPPORTED, "%s: Dk=%d, Dv=%d; supported head dims are 16, 32, 64, 128", fn, Dk, Dv);
    if (cu_seqlens) {
        if (B != 1)
            return fail(KDA_ERR_INVALID_ARG, "%s: packed sequences (cu_seqlens) need B == 1, got B=%d", fn, B);
        if (N < 1) return fail(KDA_ERR_INVALID_ARG, "%s: packed sequences need N >= 1, got N=%d", fn, N);
    } else if (N != B) {
        return fail(KDA_ERR_INVALID_ARG, "%s: without cu_seqlens N must equal B (N=%d, B=%d)", fn, N, B);
    }
    if ((int64_t)N * H > ((int64_t)1 << 26))
        return fail(KDA_ERR_UNSUPPORTED, "%s: problem too large", fn);
    if (T > 0 && (!q_raw || !k_raw || !v || !g_logit || !beta_logit || !d_o))
        return fail(KDA_ERR_INVALID_ARG, "%s: every input and d_o must be non-NULL when T > 0", fn);
    if (T > 0 && (!dq_raw || !dk_raw || !dv || !dg_logit || !dbeta_logit))
        return fail(KDA_ERR_INVALID_ARG, "%s: the token gradients must be non-NULL when T > 0", fn);
    if ((int64_t)B * T * H > ((int64_t)1 << 40))
        return fail(KDA_ERR_UNSUPPORTED, "%s: problem too large", fn);
    const bool packed = cu_seqlens != nullptr;
    const kda::PrologueBwdLayout L = kda::prologue_bwd_layout(B, T, H, Dk, Dv, N, packed);
    const size_t need = T > 0 ? (size_t)L.bytes : 0;
    if (workspace_bytes < need || (need > 0 && !workspace))
        return fail(KDA_ERR_INVALID_ARG, "%s: workspace of %zu bytes needed, got %zu%s", fn, need, workspace_bytes,
                    workspace ? "" : " (NULL)");
    if (T > 0) {
        const void* ins[] = {q_raw, k_raw, v, g_logit, beta_logit, d_o, workspace, A_log, dt_bias};
        const void* outs[] = {dq_raw, dk_raw, dv, dg_logit, dbeta_logit, dA_log, ddt_bias};
        for (const void* o : outs)
            for (const void* i : ins)
                if (o == i) return fail(KDA_ERR_INVALID_ARG, "%s: gradients must not alias an input", fn);
    }
    char* ws = static_cast<char*>(workspace);
    kda::PrologueBwdArgs p;
    p.q_raw = q_raw; p.k_raw = k_raw; p.g_logit = g_logit; p.beta_logit = beta_logit; p.v = v; p.d_o = d_o;
    p.A_log = A_log; p.dt_bias = dt_bias; p.gate_lb = gate_lower_bound; p.l2_eps = l2_eps;
    p.qf = reinterpret_cast<float*>(ws + L.qf); p.kf = reinterpret_cast<float*>(ws + L.kf);
    p.gf = reinterpret_cast<float*>(ws + L.gf); p.bf = reinterpret_cast<float*>(ws + L.bf);
    p.vf = reinterpret_cast<float*>(ws + L.vf); p.dof = reinterpret_cast<float*>(ws + L.dof);
    p.dq = dq_raw; p.dk = dk_raw; p.dg = dg_logit; p.dbeta = dbeta_logit;
    p.part_b = reinterpret_cast<float*>(ws + L.part_b); p.part_A = reinterpret_cast<float*>(ws + L.part_A);
    p.d_A_log = dA_log; p.d_dt_bias = ddt_bias;
    p.B = B; p.T = T; p.H = H; p.Dk = Dk; p.Dv = Dv; p.bf16 = dtype == KDA_BF16;
    kda::BwdArgs a;
    a.q = p.qf; a.k = p.kf; a.v = p.vf; a.g = p.gf; a.beta = p.bf; a.d_o = p.dof;
    a.s0 = initial_state; a.cu = cu_seqlens; a.d_final = d_final_state;
    a.ws = reinterpret_cast<float*>(ws + L.core);
    a.dq = dq_raw; a.dk = dk_raw; a.dv = dv; a.dg = dg_logit; a.dbeta = dbeta_logit; a.d_s0 = d_initial_state;
    a.B = B; a.T = T; a.H = H; a.Dk = Dk; a.Dv = Dv; a.N = N; a.scale = scale; a.bf16 = false;
    a.g_ge_m5 = gate_lower_bound >= -5.f;   // g lies in (gate_lower_bound, 0)
    // v and dO are read as given by the matrix-core backward (bf16 widens exactly) and by
    // either backward when already float32; only bf16 ones bound for the vector-ALU backward
    // are widened into the workspace.
    p.widen_x = dtype == KDA_BF16 && !kda::chunk_bwd_mfma_supported(a);
    if (!p.widen_x) {
        a.v = v;
        a.d_o = d_o;
        a.x_bf16 = dtype == KDA_BF16;
    }
    if ((int64_t)N * H == 0) return KDA_OK;
    const hipError_t e = kda::launch_prologue_bwd(p, a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return KDA_OK;
}

}  // extern "C"

namespace {

// The backward-from-convolution-inputs workspace: the recomputed convolution
// outputs (dtype), the gradients of them (float32), then one region that the
// prologue backward and, after it, each convolution backward use in turn.
struct BwdConvLayout {
    int64_t y[3], dy[3], rest, bytes;
};
BwdConvLayout bwd_conv_layout(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t N, bool packed,
                              kda_dtype dtype) {
    auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
    const int64_t rows = (int64_t)B * T * H;
    const int64_t elem = dtype == KDA_BF16 ? 2 : 4;
    const int64_t D[3] = {Dk, Dk, Dv};
    BwdConvLayout L;
    int64_t off = 0;
    for (int j = 0; j < 3; ++j) { L.y[j] = off; off += up(rows * D[j] * elem); }
    for (int j = 0; j < 3; ++j) { L.dy[j] = off; off += up(rows * D[j] * 4); }
    L.rest = off;
    int64_t rest = kda::prologue_bwd_layout(B, T, H, Dk, Dv, N, packed).bytes;
    for (int j = 0; j < 3; ++j)
        rest = std::max<int64_t>(rest, kda::short_conv_bwd_blocks(B, T) * (int64_t)H * D[j] * 4 * 4);
    L.bytes = off + up(rest);
    return L;
}

}  // namespace

extern "C" {

size_t kda_chunk_bwd_conv_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t N,
                                          int32_t packed, kda_dtype dtype) {
    if (B < 1 || T <= 0 || H < 1 || !dim_ok(Dk) || !dim_ok(Dv) || N < 0 || (dtype != KDA_F32 && dtype != KDA_BF16))
        return 0;
    return (size_t)bwd_conv_layout(B, T, H, Dk, Dv, N, packed != 0, dtype).bytes;
}

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
                              float* d_initial_state, void* stream) {
    g_last_error[0] = 0;
    const char* fn = "kda_chunk_bwd_conv";
    const void* x[3] = {xq, xk, xv};
    const float* w[3] = {wq, wk, wv};
    const float* s0[3] = {conv_state_q, conv_state_k, conv_state_v};
    const float* dfin[3] = {d_conv_final_q, d_conv_final_k, d_conv_final_v};
    float* dx[3] = {dxq, dxk, dxv};
    float* dw[3] = {dwq, dwk, dwv};
    float* ds0[3] = {d_conv_state_q, d_conv_state_k, d_conv_state_v};
    if (activation != 0 && activation != 1)
        return fail(KDA_ERR_INVALID_ARG, "%s: activation must be 0 (none) or 1 (SiLU), got %d", fn, activation);
    for (int j = 0; j < 3; ++j) {
        if (!w[j] || !dw[j])
            return fail(KDA_ERR_INVALID_ARG, "%s: the taps and their gradients must be non-NULL", fn);
        if (reinterpret_cast<uintptr_t>(w[j]) % 16 != 0)
            return fail(KDA_ERR_INVALID_ARG, "%s: the taps must be 16-byte aligned", fn);
        if (T > 0 && (!x[j] || !dx[j]))
            return fail(KDA_ERR_INVALID_ARG, "%s: xq, xk, xv and their gradients must be non-NULL when T > 0", fn);
    }
    if (!A_log || !dt_bias || !dA_log || !ddt_bias)
        return fail(KDA_ERR_INVALID_ARG, "%s: A_log, dt_bias, dA_log and ddt_bias must be non-NULL", fn);
    if (!(gate_lower_bound < 0.f) || !(gate_lower_bound > -1e30f))
        return fail(KDA_ERR_INVALID_ARG, "%s: gate_lower_bound must be finite and negative (got %g)", fn,
                    (double)gate_lower_bound);
    if (!(l2_eps > 0.f) || !(l2_eps < 1e30f))
        return fail(KDA_ERR_INVALID_ARG, "%s: l2_eps must be finite and positive (got %g)", fn, (double)l2_eps);
    if (B < 1 || T < 0 || H < 1 || N < 0)
        return fail(KDA_ERR_INVALID_ARG, "%s: need B >= 1, T >= 0, H >= 1, N >= 0 (got B=%d T=%d H=%d N=%d)",
                    fn, B, T, H, N);
    if (dtype != KDA_F32 && dtype != KDA_BF16)
        return fail(KDA_ERR_UNSUPPORTED, "%s: dtype %d is not KDA_F32 or KDA_BF16", fn, (int)dtype);
    if (!dim_ok(Dk) || !dim_ok(Dv))
        return fail(KDA_ERR_UNSUPPORTED, "%s: Dk=%d, Dv=%d; supported head dims are 16, 32, 64, 128", fn, Dk, Dv);
    if (cu_seqlens) {
        if (B != 1)
            return fail(KDA_ERR_INVALID_ARG, "%s: packed sequences (cu_seqlens) need B == 1, got B=%d", fn, B);
        if (N < 1) return fail(KDA_ERR_INVALID_ARG, "%s: packed sequences need N >= 1, got N=%d", fn, N);
    } else if (N != B) {
        return fail(KDA_ERR_INVALID_ARG, "%s: without cu_seqlens N must equal B (N=%d, B=%d)", fn, N, B);
    }
    if ((int64_t)N * H > ((int64_t)1 << 26) || (int64_t)B * T * H > ((int64_t)1 << 40) ||
        (int64_t)B * T > ((int64_t)1 << 31) * 16 || (int64_t)H * 128 > ((int64_t)1 << 22))
        return fail(KDA_ERR_UNSUPPORTED, "%s: problem too large", fn);
    if (T > 0 && (!g_logit || !beta_logit || !d_o || !dg_logit || !dbeta_logit))
        return fail(KDA_ERR_INVALID_ARG, "%s: every input, d_o and the token gradients must be non-NULL when T > 0",
                    fn);
    const bool packed = cu_seqlens != nullptr;
    const BwdConvLayout L = bwd_conv_layout(B, T, H, Dk, Dv, N, packed, dtype);
    const size_t need = T > 0 ? (size_t)L.bytes : 0;
    if (workspace_bytes < need || (need > 0 && !workspace))
        return fail(KDA_ERR_INVALID_ARG, "%s: workspace of %zu bytes needed, got %zu%s", fn, need, workspace_bytes,
                    workspace ? "" : " (NULL)");
    {
        const void* ins[] = {xq, xk, xv, wq, wk, wv, conv_state_q, conv_state_k, conv_state_v, g_logit, beta_logit,
                             A_log, dt_bias, initial_state, d_o, d_final_state, d_conv_final_q, d_conv_final_k,
                             d_conv_final_v, workspace};
        const void* outs[] = {dxq, dxk, dxv, dwq, dwk, dwv, d_conv_state_q, d_conv_state_k, d_conv_state_v,
                              dg_logit, dbeta_logit, dA_log, ddt_bias, d_initial_state};
        for (const void* o : outs)
            for (const void* i : ins)
                if (o && o == i) return fail(KDA_ERR_INVALID_ARG, "%s: gradients must not alias an input", fn);
    }
    char* ws = static_cast<char*>(workspace);
    void* y[3] = {nullptr, nullptr, nullptr};
    float* dy[3] = {nullptr, nullptr, nullptr};
    if (T > 0) {
        for (int j = 0; j < 3; ++j) {
            y[j] = ws + L.y[j];
            dy[j] = reinterpret_cast<float*>(ws + L.dy[j]);
        }
        // the forward's convolutions again, into the workspace
        kda::ConvArgs c[3];
        const int32_t D[3] = {Dk, Dk, Dv};
        for (int j = 0; j < 3; ++j) {
            c[j].x = x[j]; c[j].w = w[j]; c[j].state_in = s0[j]; c[j].cu = cu_seqlens; c[j].y = y[j];
            c[j].state_out = nullptr; c[j].B = B; c[j].T = T; c[j].C = H * D[j]; c[j].N = N;
            c[j].act = activation == 1; c[j].bf16 = dtype == KDA_BF16;
        }
        const hipError_t e = kda::launch_short_conv_set(c, 3, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    }
    void* rest = T > 0 ? ws + L.rest : nullptr;
    const size_t rest_bytes = T > 0 ? (size_t)(L.bytes - L.rest) : 0;
    char inner[sizeof(g_last_error)];
    kda_status st = kda_chunk_bwd_prologue(y[0], y[1], y[2], g_logit, beta_logit, A_log, dt_bias, gate_lower_bound,
                                           l2_eps, initial_state, cu_seqlens, d_o, d_final_state, B, T, H, Dk, Dv, N,
                                           scale, dtype, rest, rest_bytes, dy[0], dy[1], dy[2], dg_logit, dbeta_logit,
                                           dA_log, ddt_bias, d_initial_state, stream);
    if (st != KDA_OK) {
        snprintf(inner, sizeof(inner), "%s", g_last_error);
        return fail(st, "%s: %s", fn, inner);
    }
    const int32_t D[3] = {Dk, Dk, Dv};
    for (int j = 0; j < 3; ++j) {
        st = kda_short_conv_bwd(x[j], w[j], s0[j], cu_seqlens, dy[j], dfin[j], B, T, H * D[j], N, activation, dtype,
                                rest, rest_bytes, dx[j], dw[j], ds0[j], stream);
        if (st != KDA_OK) {
            snprintf(inner, sizeof(inner), "%s", g_last_error);
            return fail(st, "%s: %s", fn, inner);
        }
    }
    return KDA_OK;
}

kda_status kda_prologue(const void* q_raw, const void* k_raw, const void* g_logit, const void* beta_logit,
                        const float* A_log, const float* dt_bias, float gate_lower_bound, float l2_eps, int32_t B,
                        int32_t T, int32_t H, int32_t Dk, kda_dtype dtype, void* q, void* k, void* g, void* beta,
                        void* stream) {
    g_last_error[0] = 0;
    const char* fn = "kda_prologue";
    if (B < 1 || T < 0 || H < 1)
        return fail(KDA_ERR_INVALID_ARG, "%s: need B >= 1, T >= 0, H >= 1 (got B=%d T=%d H=%d)", fn, B, T, H);
    if (dtype != KDA_F32 && dtype != KDA_BF16)
        return fail(KDA_ERR_UNSUPPORTED, "%s: dtype %d is not KDA_F32 or KDA_BF16", fn, (int)dtype);
    if (!dim_ok(Dk)) return fail(KDA_ERR_UNSUPPORTED, "%s: Dk=%d; supported head dims are 16, 32, 64, 128", fn, Dk);
    if ((int64_t)B * T * H > ((int64_t)1 << 40)) return fail(KDA_ERR_UNSUPPORTED, "%s: problem too large", fn);
    if (T > 0 && (!q_raw || !k_raw || !g_logit || !beta_logit || !q || !k || !g || !beta || !A_log || !dt_bias))
        return fail(KDA_ERR_INVALID_ARG, "%s: every input and output must be non-NULL when T > 0", fn);
    if (!(gate_lower_bound < 0.f) || !(gate_lower_bound > -1e30f))
        return fail(KDA_ERR_INVALID_ARG, "%s: gate_lower_bound must be finite and negative (got %g)", fn,
                    (double)gate_lower_bound);
    if (!(l2_eps > 0.f) || !(l2_eps < 1e30f))
        return fail(KDA_ERR_INVALID_ARG, "%s: l2_eps must be finite and positive (got %g)", fn, (double)l2_eps);
    if (T == 0) return KDA_OK;
    {
        // an output may be its own input (in place), and nothing else
        const void* ins[] = {q_raw, k_raw, g_logit, beta_logit};
        void* outs[] = {q, k, g, beta};
        for (int j = 0; j < 4; ++j) {
            for (int i = 0; i < 4; ++i)
                if (i != j && outs[j] == ins[i])
                    return fail(KDA_ERR_INVALID_ARG, "%s: an output may alias only its own input", fn);
            for (int i = 0; i < 4; ++i)
                if (i != j && outs[j] == outs[i])
                    return fail(KDA_ERR_INVALID_ARG, "%s: the outputs must be distinct", fn);
            if (outs[j] == A_log || outs[j] == dt_bias)
                return fail(KDA_ERR_INVALID_ARG, "%s: an output may alias only its own input", fn);
        }
    }
    kda::PrologueBwdArgs p{};
    p.q_raw = q_raw; p.k_raw = k_raw; p.g_logit = g_logit; p.beta_logit = beta_logit;
    p.A_log = A_log; p.dt_bias = dt_bias; p.gate_lb = gate_lower_bound; p.l2_eps = l2_eps;
    // the apply pass writes its outputs in the input dtype here
    p.qf = static_cast<float*>(q); p.kf = static_cast<float*>(k); p.gf = static_cast<float*>(g);
    p.bf = static_cast<float*>(beta);
    p.widen_x = false;
    p.B = B; p.T = T; p.H = H; p.Dk = Dk; p.Dv = Dk; p.bf16 = dtype == KDA_BF16;
    const hipError_t e = kda::launch_prologue(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return KDA_OK;
}

kda_status kda_short_conv(const void* x, const float* weight, const float* conv_state_in,
                          const int32_t* cu_seqlens, int32_t B, int32_t T, int32_t C, int32_t N,
                          int32_t activation, kda_dtype dtype, void* y, float* conv_state_out, void* stream) {
    g_last_error[0] = 0;
    const char* fn = "kda_short_conv";
    if (T > 0 && (!x || !y || !weight))
        return fail(KDA_ERR_INVALID_ARG, "%s: x, weight and y must be non-NULL when T > 0", fn);
    if (B < 1 || T < 0 || C < 1 || N < 0)
        return fail(KDA_ERR_INVALID_ARG, "%s: need B >= 1, T >= 0, C >= 1, N >= 0 (got B=%d T=%d C=%d N=%d)", fn,
                    B, T, C, N);
    if (C % 8 != 0)
        return fail(KDA_ERR_UNSUPPORTED, "%s: C=%d; the channel count must be a multiple of 8", fn, C);
    if (activation != 0 && activation != 1)
        return fail(KDA_ERR_INVALID_ARG, "%s: activation must be 0 (none) or 1 (SiLU), got %d", fn, activation);
    if (dtype != KDA_F32 && dtype != KDA_BF16)
        return fail(KDA_ERR_UNSUPPORTED, "%s: dtype %d is not KDA_F32 or KDA_BF16", fn, (int)dtype);
    if (cu_seqlens) {
        if (B != 1)
            return fail(KDA_ERR_INVALID_ARG, "%s: packed sequences (cu_seqlens) need B == 1, got B=%d", fn, B);
        if (N < 1)
            return fail(KDA_ERR_INVALID_ARG, "%s: packed sequences need N >= 1, got N=%d", fn, N);
    } else if (N != B) {
        return fail(KDA_ERR_INVALID_ARG, "%s: without cu_seqlens N must equal B (N=%d, B=%d)", fn, N, B);
    }
    if ((int64_t)B * T > ((int64_t)1 << 31) * 16 || (int64_t)C > ((int64_t)1 << 24))
        return fail(KDA_ERR_UNSUPPORTED, "%s: problem too large", fn);
    if (T > 0 && y == x)
        return fail(KDA_ERR_INVALID_ARG, "%s: y must not alias x", fn);
    kda::ConvArgs a;
    a.x = x; a.w = weight; a.state_in = conv_state_in; a.cu = cu_seqlens; a.y = y; a.state_out = conv_state_out;
    a.B = B; a.T = T; a.C = C; a.N = N; a.act = activation == 1; a.bf16 = dtype == KDA_BF16;
    if ((int64_t)B * T == 0 && !conv_state_out) return KDA_OK;
    const hipError_t e = kda::launch_short_conv(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return KDA_OK;
}

size_t kda_short_conv_bwd_workspace_bytes(int32_t B, int32_t T, int32_t C) {
    if (B < 1 || T < 0 || C < 1) return 0;
    return (size_t)kda::short_conv_bwd_blocks(B, T) * (size_t)C * 4 * sizeof(float);
}

kda_status kda_short_conv_bwd(const void* x, const float* weight, const float* conv_state_in,
                              const int32_t* cu_seqlens, const float* dy, const float* d_final_state, int32_t B,
                              int32_t T, int32_t C, int32_t N, int32_t activation, kda_dtype dtype, void* workspace,
                              size_t workspace_bytes, float* dx, float* dweight, float* d_state_in, void* stream) {
    g_last_error[0] = 0;
    const char* fn = "kda_short_conv_bwd";
    if (!weight || !dweight)
        return fail(KDA_ERR_INVALID_ARG, "%s: weight and dweight must be non-NULL", fn);
    if (T > 0 && (!x || !dy || !dx))
        return fail(KDA_ERR_INVALID_ARG, "%s: x, dy and dx must be non-NULL when T > 0", fn);
    if (B < 1 || T < 0 || C < 1 || N < 0)
        return fail(KDA_ERR_INVALID_ARG, "%s: need B >= 1, T >= 0, C >= 1, N >= 0 (got B=%d T=%d C=%d N=%d)", fn,
                    B, T, C, N);
    if (C % 8 != 0)
        return fail(KDA_ERR_UNSUPPORTED, "%s: C=%d; the channel count must be a multiple of 8", fn, C);
    if (activation != 0 && activation != 1)
        return fail(KDA_ERR_INVALID_ARG, "%s: activation must be 0 (none) or 1 (SiLU), got %d", fn, activation);
    if (dtype != KDA_F32 && dtype != KDA_BF16)
        return fail(KDA_ERR_UNSUPPORTED, "%s: dtype %d is not KDA_F32 or KDA_BF16", fn, (int)dtype);
    if (cu_seqlens) {
        if (B != 1)
            return fail(KDA_ERR_INVALID_ARG, "%s: packed sequences (cu_seqlens) need B == 1, got B=%d", fn, B);
        if (N < 1)
            return fail(KDA_ERR_INVALID_ARG, "%s: packed sequences need N >= 1, got N=%d", fn, N);
    } else if (N != B) {
        return fail(KDA_ERR_INVALID_ARG, "%s: without cu_seqlens N must equal B (N=%d, B=%d)", fn, N, B);
    }
    if ((int64_t)B * T > ((int64_t)1 << 31) * 16 || (int64_t)C > ((int64_t)1 << 22))
        return fail(KDA_ERR_UNSUPPORTED, "%s: problem too large", fn);
    const size_t need = kda_short_conv_bwd_workspace_bytes(B, T, C);
    if (workspace_bytes < need || (need > 0 && !workspace))
        return fail(KDA_ERR_INVALID_ARG, "%s: workspace of %zu bytes needed, got %zu%s", fn, need, workspace_bytes,
                    workspace ? "" : " (NULL)");
    {
        const void* ins[] = {x, weight, conv_state_in, dy, d_final_state, workspace};
        const void* outs[] = {dx, dweight, d_state_in};
        for (const void* o : outs)
            for (const void* i : ins)
                if (o && o == i) return fail(KDA_ERR_INVALID_ARG, "%s: gradients must not alias an input", fn);
    }
    kda::ConvBwdArgs a;
    a.fwd.x = x; a.fwd.w = weight; a.fwd.state_in = conv_state_in; a.fwd.cu = cu_seqlens; a.fwd.y = nullptr;
    a.fwd.state_out = nullptr; a.fwd.B = B; a.fwd.T = T; a.fwd.C = C; a.fwd.N = N; a.fwd.act = activation == 1;
    a.fwd.bf16 = dtype == KDA_BF16;
    a.dy = dy; a.d_final = d_final_state; a.dx = dx; a.dw = dweight; a.d_state = d_state_in;
    a.part = static_cast<float*>(workspace);
    a.B = B; a.T = T; a.C = C; a.N = N;
    const hipError_t e = kda::launch_short_conv_bwd(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return KDA_OK;
}

kda_status kda_short_conv_step(const void* x, const float* weight, float* conv_cache, const int32_t* cache_slots,
                               int32_t n_slots, int32_t Nb, int32_t C, int32_t activation, kda_dtype dtype,
                               void* y, void* stream) {
    g_last_error[0] = 0;
    const char* fn = "kda_short_conv_step";
    if (Nb != 0 && (!x || !weight || !conv_cache || !y))
        return fail(KDA_ERR_INVALID_ARG, "%s: x, weight, conv_cache and y must be non-NULL", fn);
    if (Nb < 0 || C < 1 || n_slots < 0)
        return fail(KDA_ERR_INVALID_ARG, "%s: need Nb >= 0, C >= 1, n_slots >= 0 (got %d, %d, %d)", fn, Nb, C,
                    n_slots);
    if (C % 8 != 0)
        return fail(KDA_ERR_UNSUPPORTED, "%s: C=%d; the channel count must be a multiple of 8", fn, C);
    if (activation != 0 && activation != 1)
        return fail(KDA_ERR_INVALID_ARG, "%s: activation must be 0 (none) or 1 (SiLU), got %d", fn, activation);
    if (dtype != KDA_F32 && dtype != KDA_BF16)
        return fail(KDA_ERR_UNSUPPORTED, "%s: dtype %d is not KDA_F32 or KDA_BF16", fn, (int)dtype);
    if (!cache_slots && Nb > n_slots)
        return fail(KDA_ERR_INVALID_ARG, "%s: without cache_slots row r uses slot r, so Nb (%d) must be <= n_slots (%d)",
                    fn, Nb, n_slots);
    if ((int64_t)C > ((int64_t)1 << 24))
        return fail(KDA_ERR_UNSUPPORTED, "%s: C too large", fn);
    if (Nb == 0) return KDA_OK;
    if (y == x) return fail(KDA_ERR_INVALID_ARG, "%s: y must not alias x", fn);
    kda::ConvStepArgs a;
    a.x = x; a.w = weight; a.cache = conv_cache; a.slots = cache_slots; a.y = y;
    a.n_slots = n_slots; a.Nb = Nb; a.C = C; a.act = activation == 1; a.bf16 = dtype == KDA_BF16;
    const hipError_t e = kda::launch_short_conv_step(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return KDA_OK;
}

kda_status kda_recurrent_step(const void* q, const void* k, const void* v, const void* g,
                              const void* beta, float* state_cache, const int32_t* state_slots,
                              int32_t n_slots, int32_t Nb, int32_t H, int32_t Dk, int32_t Dv,
                              float scale, kda_dtype dtype, void* o, void* stream) {
    g_last_error[0] = 0;
    const char* fn = "kda_recurrent_step";
    kda::StepArgs a;
    const kda_status st = check_step(fn, q, k, v, g, beta, state_cache, state_slots, n_slots, Nb, H, Dk, Dv, scale,
                                     dtype, o, a);
    if (st != KDA_OK || Nb == 0) return st;
    return launch_step(fn, a, stream);
}

kda_status kda_recurrent_step_prologue(const void* q_raw, const void* k_raw, const void* v, const void* g_logit,
                                       const void* beta_logit, const float* A_log, const float* dt_bias,
                                       float gate_lower_bound, float l2_eps, float* state_cache,
                                       const int32_t* state_slots, int32_t n_slots, int32_t Nb, int32_t H,
                                       int32_t Dk, int32_t Dv, float scale, kda_dtype dtype, void* o,
                                       void* stream) {
    g_last_error[0] = 0;
    const char* fn = "kda_recurrent_step_prologue";
    kda::StepArgs a;
    kda_status st = check_step(fn, q_raw, k_raw, v, g_logit, beta_logit, state_cache, state_slots, n_slots, Nb, H,
                               Dk, Dv, scale, dtype, o, a);
    if (st == KDA_OK) st = check_step_prologue(fn, A_log, dt_bias, gate_lower_bound, l2_eps, Nb, a);
    if (st != KDA_OK || Nb == 0) return st;
    return launch_step(fn, a, stream);
}

kda_status kda_recurrent_step_conv(const void* xq, const void* xk, const void* xv, const float* wq,
                                   const float* wk, const float* wv, float* conv_cache_q, float* conv_cache_k,
                                   float* conv_cache_v, int32_t activation, const void* g_logit,
                                   const void* beta_logit, const float* A_log, const float* dt_bias,
                                   float gate_lower_bound, float l2_eps, float* state_cache,
                                   const int32_t* state_slots, int32_t n_slots, int32_t Nb, int32_t H, int32_t Dk,
                                   int32_t Dv, float scale, kda_dtype dtype, void* o, void* stream) {
    g_last_error[0] = 0;
    const char* fn = "kda_recurrent_step_conv";
    kda::StepArgs a;
    kda_status st = check_step(fn, xq, xk, xv, g_logit, beta_logit, state_cache, state_slots, n_slots, Nb, H, Dk,
                               Dv, scale, dtype, o, a);
    if (st == KDA_OK) st = check_step_prologue(fn, A_log, dt_bias, gate_lower_bound, l2_eps, Nb, a);
    if (st != KDA_OK) return st;
    if (activation != 0 && activation != 1)
        return fail(KDA_ERR_INVALID_ARG, "%s: activation must be 0 (none) or 1 (SiLU), got %d", fn, activation);
    if (Nb == 0) return KDA_OK;
    const float* w[3] = {wq, wk, wv};
    float* cache[3] = {conv_cache_q, conv_cache_k, conv_cache_v};
    for (int j = 0; j < 3; ++j) {
        if (!w[j] || !cache[j])
            return fail(KDA_ERR_INVALID_ARG, "%s: the taps and convolution caches must be non-NULL", fn);
        if (reinterpret_cast<uintptr_t>(w[j]) % 16 != 0)
            return fail(KDA_ERR_INVALID_ARG, "%s: the taps must be 16-byte aligned", fn);
    }
    if (cache[0] == cache[1] || cache[0] == cache[2] || cache[1] == cache[2] || cache[0] == state_cache ||
        cache[1] == state_cache || cache[2] == state_cache)
        return fail(KDA_ERR_INVALID_ARG, "%s: the convolution caches and the state cache must be distinct", fn);
    for (int j = 0; j < 3; ++j) {
        if (cache[j] == o)
            return fail(KDA_ERR_INVALID_ARG, "%s: o must not alias an input", fn);
        a.conv_w[j] = w[j];
        a.conv_cache[j] = cache[j];
    }
    a.conv = true;
    a.conv_act = activation == 1;
    return launch_step(fn, a, stream);
}

}  // extern "C"
