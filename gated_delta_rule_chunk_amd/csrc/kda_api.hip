// C ABI of libkda.so: argument validation, kernel selection, error mapping.
// Every check runs on the host before any launch; a rejected call touches no
// memory and makes no HIP call.
#include <stdarg.h>
#include <stdio.h>

#include "../../include/kda.h"
#include "launchers.hpp"

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

}  // namespace

extern "C" {

const char* kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
        case KDA_ERR_HIP: return "KDA_ERR_HIP";
    }
    return "KDA_UNKNOWN_STATUS";
}

const char* kda_last_error_message(void) { return g_last_error; }

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const void* g,
                         const void* beta, const float* initial_state,
                         const int32_t* cu_seqlens, int32_t B, int32_t T, int32_t H,
                         int32_t Dk, int32_t Dv, int32_t N, int32_t chunk_size, float scale,
                         kda_dtype dtype, void* o, float* final_state, void* stream) {
    g_last_error[0] = 0;
    if (T > 0 && (!q || !k || !v || !g || !beta || !o))
        return fail(KDA_ERR_INVALID_ARG, "kda_chunk_fwd: q, k, v, g, beta and o must be non-NULL when T > 0");
    if (B < 1 || T < 0 || H < 1 || N < 0)
        return fail(KDA_ERR_INVALID_ARG, "kda_chunk_fwd: need B >= 1, T >= 0, H >= 1, N >= 0 (got B=%d T=%d H=%d N=%d)",
                    B, T, H, N);
    if (dtype != KDA_F32 && dtype != KDA_BF16)
        return fail(KDA_ERR_UNSUPPORTED, "kda_chunk_fwd: dtype %d is not KDA_F32 or KDA_BF16", (int)dtype);
    if (!dim_ok(Dk) || !dim_ok(Dv))
        return fail(KDA_ERR_UNSUPPORTED, "kda_chunk_fwd: Dk=%d, Dv=%d; supported head dims are 16, 32, 64, 128",
                    Dk, Dv);
    const int32_t chunk = chunk_size == 0 ? 64 : chunk_size;
    if (chunk != 16 && chunk != 32 && chunk != 64)
        return fail(KDA_ERR_UNSUPPORTED, "kda_chunk_fwd: chunk_size=%d; supported are 16, 32, 64 (0 = 64)",
                    chunk_size);
    if (cu_seqlens) {
        if (B != 1)
            return fail(KDA_ERR_INVALID_ARG, "kda_chunk_fwd: packed sequences (cu_seqlens) need B == 1, got B=%d", B);
        if (N < 1)
            return fail(KDA_ERR_INVALID_ARG, "kda_chunk_fwd: packed sequences need N >= 1, got N=%d", N);
    } else if (N != B) {
        return fail(KDA_ERR_INVALID_ARG, "kda_chunk_fwd: without cu_seqlens N must equal B (N=%d, B=%d)", N, B);
    }
    const int64_t units = (int64_t)N * H;
    if (units > (int64_t)1 << 26 || (int64_t)B * T * H > ((int64_t)1 << 40))
        return fail(KDA_ERR_UNSUPPORTED, "kda_chunk_fwd: problem too large (N*H=%lld)", (long long)units);
    if (T > 0 && (o == q || o == k || o == v || o == g || o == beta))
        return fail(KDA_ERR_INVALID_ARG, "kda_chunk_fwd: o must not alias an input");

    kda::ChunkArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.s0 = initial_state; a.cu = cu_seqlens; a.o = o; a.sT = final_state;
    a.B = B; a.T = T; a.H = H; a.Dk = Dk; a.Dv = Dv; a.N = N; a.chunk = chunk;
    a.scale = scale; a.bf16 = dtype == KDA_BF16;
    if (units == 0) return KDA_OK;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = kda::chunk_mfma_supported(a) ? kda::launch_chunk_mfma(a, s)
                                                      : kda::launch_chunk_generic(a, s);
    if (e != hipSuccess)
        return fail(KDA_ERR_HIP, "kda_chunk_fwd: launch failed: %s", hipGetErrorString(e));
    return KDA_OK;
}

kda_status kda_recurrent_step(const void* q, const void* k, const void* v, const void* g,
                              const void* beta, float* state_cache, const int32_t* state_slots,
                              int32_t n_slots, int32_t Nb, int32_t H, int32_t Dk, int32_t Dv,
                              float scale, kda_dtype dtype, void* o, void* stream) {
    g_last_error[0] = 0;
    if (Nb != 0 && (!q || !k || !v || !g || !beta || !state_cache || !o))
        return fail(KDA_ERR_INVALID_ARG,
                    "kda_recurrent_step: q, k, v, g, beta, state_cache and o must be non-NULL");
    if (Nb < 0 || H < 1 || n_slots < 0)
        return fail(KDA_ERR_INVALID_ARG, "kda_recurrent_step: need Nb >= 0, H >= 1, n_slots >= 0 (got %d, %d, %d)",
                    Nb, H, n_slots);
    if (dtype != KDA_F32 && dtype != KDA_BF16)
        return fail(KDA_ERR_UNSUPPORTED, "kda_recurrent_step: dtype %d is not KDA_F32 or KDA_BF16", (int)dtype);
    if (!dim_ok(Dk) || !dim_ok(Dv))
        return fail(KDA_ERR_UNSUPPORTED, "kda_recurrent_step: Dk=%d, Dv=%d; supported head dims are 16, 32, 64, 128",
                    Dk, Dv);
    if (!state_slots && Nb > n_slots)
        return fail(KDA_ERR_INVALID_ARG, "kda_recurrent_step: without state_slots row r uses slot r, so Nb (%d) must be <= n_slots (%d)",
                    Nb, n_slots);
    if ((int64_t)Nb * H > ((int64_t)1 << 30))
        return fail(KDA_ERR_UNSUPPORTED, "kda_recurrent_step: Nb*H too large");
    if (Nb == 0) return KDA_OK;
    if (o == q || o == k || o == v || o == g || o == beta || o == state_cache)
        return fail(KDA_ERR_INVALID_ARG, "kda_recurrent_step: o must not alias an input");

    kda::StepArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.cache = state_cache; a.slots = state_slots; a.o = o;
    a.Nb = Nb; a.H = H; a.Dk = Dk; a.Dv = Dv; a.scale = scale; a.bf16 = dtype == KDA_BF16;
    const hipError_t e = kda::launch_recurrent_step(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(KDA_ERR_HIP, "kda_recurrent_step: launch failed: %s", hipGetErrorString(e));
    return KDA_OK;
}

}  // extern "C"
