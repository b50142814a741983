// Short causal depthwise convolution over time (kernel 4) of the q, k or v
// projections, with a per-sequence conv state, and its decode step.
//
// Per sequence and channel c, with the window ending at token t:
//   y[t][c] = sum_{i=0..3} w[c][i] * x[t - 3 + i][c]
// where the three inputs before the sequence's first token come from the conv
// state ([N][3][C]: x[-3], x[-2], x[-1]) or are zero; with the activation,
// y <- y * sigmoid(y). The final state is the window's last three inputs.
//
// The kernels are bandwidth-bound: a lane owns a few consecutive channels, a
// wave walks a run of consecutive tokens keeping the three previous inputs in
// registers, so every wave access is contiguous across lanes and every input
// is read once (plus a three-token halo per run).
#include <algorithm>

#include "device_common.hpp"
#include "launchers.hpp"

namespace kda {
namespace {

constexpr int kThreadsConv = 256;

// Up to kMaxConvSet convolutions of one layer's projections (same dtype,
// activation, B, T and N; C may differ) in one launch: blockIdx.z picks the
// projection.
struct ConvSet {
    ConvArgs p[kMaxConvSet];
};

template <typename T> struct Vec8;
template <> struct Vec8<__bf16> {
    static __device__ __forceinline__ void load(const __bf16* p, float (&f)[8]) {
        unpack8(*reinterpret_cast<const uint4*>(p), f);
    }
    static __device__ __forceinline__ void store(__bf16* p, const float (&f)[8]) {
        uint4 u;
        u.x = pack2_bf16(f[0], f[1]);
        u.y = pack2_bf16(f[2], f[3]);
        u.z = pack2_bf16(f[4], f[5]);
        u.w = pack2_bf16(f[6], f[7]);
        *reinterpret_cast<uint4*>(p) = u;
    }
};
template <> struct Vec8<float> {
    static __device__ __forceinline__ void load(const float* p, float (&f)[8]) {
        const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    }
    static __device__ __forceinline__ void store(float* p, const float (&f)[8]) {
        reinterpret_cast<float4*>(p)[0] = float4{f[0], f[1], f[2], f[3]};
        reinterpret_cast<float4*>(p)[1] = float4{f[4], f[5], f[6], f[7]};
    }
};

__device__ __forceinline__ void load_state8(const float* p, float (&f)[8]) { Vec8<float>::load(p, f); }

template <bool kAct>
__device__ __forceinline__ float activate(float y) {
    if constexpr (kAct) return y * __builtin_amdgcn_rcpf(1.f + __expf(-y));
    return y;
}

// The sequence holding flattened token t: [bos, eos) and its index n.
__device__ __forceinline__ void find_sequence(const ConvArgs& a, int64_t t, int& n, int64_t& bos, int64_t& eos) {
    if (a.cu) {
        int lo = 0, hi = a.N;            // invariant: cu[lo] <= t < cu[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.cu[mid] <= t) lo = mid; else hi = mid;
        }
        n = lo;
        bos = a.cu[lo];
        eos = a.cu[lo + 1];
    } else {
        n = (int)(t / a.T);
        bos = (int64_t)n * a.T;
        eos = bos + a.T;
    }
}


// Prefill: a lane owns kFwdCh channels; a wave walks kFwdWaveRows
// consecutive tokens once, carrying the last three inputs of the window, and
// goes in groups of up to kFwdGroup tokens with every load of the group
// issued before any is used. The wave's token range and the sequence bounds
// are uniform across the wave. The four waves of a workgroup take
// consecutive token ranges of the same channels.
// Tiling measured at T=4096, C=12288, bf16: 4 channels per lane and 64
// tokens per wave, in groups of 16 tokens (4% faster than groups of 8, as
// fast as 32; 8 channels per lane, 32- or 128-token runs and 2-token groups
// are slower). The group's loads are what is in flight: 8 KiB per wave at
// four waves per SIMD. Capping the registers for more waves spills and
// halves the rate.
constexpr int kFwdCh = 4;
constexpr int kFwdWaveRows = 64;
constexpr int kFwdBlockRows = 4 * kFwdWaveRows;
constexpr int kFwdBlockCh = 64 * kFwdCh;
constexpr int kFwdGroup = 16;
typedef uint32_t ntu2 __attribute__((ext_vector_type(2)));
typedef float ntf4 __attribute__((ext_vector_type(4)));

// Four-channel accesses (the streaming kernels' unit). Loads are
// non-temporal: every input element is read once (the halo rows a second time
// by the neighbouring wave). Stores keep the default policy, since the
// forward's outputs are read right after by the chunk kernel, except
// store_nt, for outputs that nothing reads soon (the backward's dx).
template <typename T, int N> struct LoadN;
template <typename T> struct LoadN<T, 8> {
    static __device__ __forceinline__ void load(const T* p, float (&f)[8]) { Vec8<T>::load(p, f); }
    static __device__ __forceinline__ void store(T* p, const float (&f)[8]) { Vec8<T>::store(p, f); }
};
template <> struct LoadN<float, 4> {
    static __device__ __forceinline__ void load(const float* p, float (&f)[4]) {
        const ntf4 a = __builtin_nontemporal_load(reinterpret_cast<const ntf4*>(p));
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    }
    static __device__ __forceinline__ void store(float* p, const float (&f)[4]) {
        *reinterpret_cast<float4*>(p) = float4{f[0], f[1], f[2], f[3]};
    }
    static __device__ __forceinline__ void store_nt(float* p, const float (&f)[4]) {
        __builtin_nontemporal_store(ntf4{f[0], f[1], f[2], f[3]}, reinterpret_cast<ntf4*>(p));
    }
};
template <> struct LoadN<__bf16, 4> {
    static __device__ __forceinline__ void load(const __bf16* p, float (&f)[4]) {
        const ntu2 u = __builtin_nontemporal_load(reinterpret_cast<const ntu2*>(p));
        f[0] = __uint_as_float(u.x << 16); f[1] = __uint_as_float(u.x & 0xffff0000u);
        f[2] = __uint_as_float(u.y << 16); f[3] = __uint_as_float(u.y & 0xffff0000u);
    }
    static __device__ __forceinline__ void store(__bf16* p, const float (&f)[4]) {
        uint2 u;
        u.x = pack2_bf16(f[0], f[1]);
        u.y = pack2_bf16(f[2], f[3]);
        *reinterpret_cast<uint2*>(p) = u;
    }
};

// input x[tau] of sequence n (tau relative to its start, tau >= -3), N channels
template <typename T, int N>
__device__ __forceinline__ void window_input_n(const ConvArgs& a, const T* x, int n, int64_t bos, int64_t tau,
                                               int64_t c0, float (&f)[N]) {
    if (tau >= 0) {
        LoadN<T, N>::load(x + (bos + tau) * a.C + c0, f);
    } else if (a.state_in) {
        LoadN<float, N>::load(a.state_in + ((int64_t)n * 3 + (3 + tau)) * a.C + c0, f);
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) f[i] = 0.f;
    }
}

template <typename T, bool kAct, int G>
__device__ __forceinline__ void conv_fwd_group(const ConvArgs& a, const T* x, T* y, int64_t c0, int64_t u,
                                               const float (&w)[kFwdCh][4], float (&h0)[kFwdCh],
                                               float (&h1)[kFwdCh], float (&h2)[kFwdCh]) {
    float xu[G][kFwdCh];
#pragma unroll
    for (int j = 0; j < G; ++j) LoadN<T, kFwdCh>::load(x + (u + j) * a.C + c0, xu[j]);
#pragma unroll
    for (int j = 0; j < G; ++j) {
        float out[kFwdCh];
#pragma unroll
        for (int i = 0; i < kFwdCh; ++i) {
            out[i] = activate<kAct>(fmaf(w[i][3], xu[j][i], fmaf(w[i][2], h2[i], fmaf(w[i][1], h1[i], w[i][0] * h0[i]))));
            h0[i] = h1[i];
            h1[i] = h2[i];
            h2[i] = xu[j][i];
        }
        LoadN<T, kFwdCh>::store(y + (u + j) * a.C + c0, out);
    }
}

template <typename T, bool kAct>
__global__ __launch_bounds__(256) void short_conv_kernel(ConvSet set) {
    const ConvArgs& a = set.p[blockIdx.z];   // the projection
    if (!a.y) return;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t c0 = (int64_t)blockIdx.y * kFwdBlockCh + (int64_t)lane * kFwdCh;
    const int64_t BT = (int64_t)a.B * a.T;
    const int64_t tb = (int64_t)blockIdx.x * kFwdBlockRows + (int64_t)wv * kFwdWaveRows;
    if (c0 >= a.C || tb >= BT) return;
    const int64_t te = tb + kFwdWaveRows < BT ? tb + kFwdWaveRows : BT;
    const T* x = static_cast<const T*>(a.x);
    T* y = static_cast<T*>(a.y);
    float w[kFwdCh][4];
#pragma unroll
    for (int i = 0; i < kFwdCh; ++i) {
        const float4 wi = reinterpret_cast<const float4*>(a.w)[c0 + i];
        w[i][0] = wi.x; w[i][1] = wi.y; w[i][2] = wi.z; w[i][3] = wi.w;
    }
    int n;
    int64_t bos, eos;
    find_sequence(a, tb, n, bos, eos);
    float h0[kFwdCh], h1[kFwdCh], h2[kFwdCh];      // x[u-3], x[u-2], x[u-1]
    window_input_n<T, kFwdCh>(a, x, n, bos, tb - bos - 3, c0, h0);
    window_input_n<T, kFwdCh>(a, x, n, bos, tb - bos - 2, c0, h1);
    window_input_n<T, kFwdCh>(a, x, n, bos, tb - bos - 1, c0, h2);
    int64_t u = tb;
    while (u < te) {
        if (u == eos) {
            // the next non-empty sequence starts here: its window starts from its state
            find_sequence(a, u, n, bos, eos);
            window_input_n<T, kFwdCh>(a, x, n, bos, -3, c0, h0);
            window_input_n<T, kFwdCh>(a, x, n, bos, -2, c0, h1);
            window_input_n<T, kFwdCh>(a, x, n, bos, -1, c0, h2);
        }
        const int64_t rem = (eos < te ? eos : te) - u;
        if (rem >= kFwdGroup) {
            conv_fwd_group<T, kAct, kFwdGroup>(a, x, y, c0, u, w, h0, h1, h2);
            u += kFwdGroup;
        } else if (rem >= 4) {
            conv_fwd_group<T, kAct, 4>(a, x, y, c0, u, w, h0, h1, h2);
            u += 4;
        } else if (rem == 3) {
            conv_fwd_group<T, kAct, 3>(a, x, y, c0, u, w, h0, h1, h2);
            u += 3;
        } else if (rem == 2) {
            conv_fwd_group<T, kAct, 2>(a, x, y, c0, u, w, h0, h1, h2);
            u += 2;
        } else {
            conv_fwd_group<T, kAct, 1>(a, x, y, c0, u, w, h0, h1, h2);
            u += 1;
        }
    }
}

// Final conv state of every sequence: its window's last three inputs. One
// thread per (sequence, 8 channels) reads all three before writing, so the
// output may alias the input state.
template <typename T>
__global__ __launch_bounds__(kThreadsConv) void short_conv_state_kernel(ConvSet set) {
    const ConvArgs& a = set.p[blockIdx.z];   // the projection
    const int64_t c0 = ((int64_t)blockIdx.y * kThreadsConv + threadIdx.x) * 8;
    const int n = blockIdx.x;
    if (!a.state_out || c0 >= a.C) return;
    int64_t bos, eos;
    if (a.cu) {
        bos = a.cu[n];
        eos = a.cu[n + 1];
    } else {
        bos = (int64_t)n * a.T;
        eos = bos + a.T;
    }
    const T* x = static_cast<const T*>(a.x);
    const int64_t L = eos - bos;
    float f[3][8];
#pragma unroll
    for (int j = 0; j < 3; ++j) window_input_n<T, 8>(a, x, n, bos, L - 3 + j, c0, f[j]);
#pragma unroll
    for (int j = 0; j < 3; ++j) Vec8<float>::store(a.state_out + ((int64_t)n * 3 + j) * a.C + c0, f[j]);
}

// Decode: row r reads and shifts cache[slot(r)] ([3][C]); a row whose slot
// lies outside [0, n_slots) is padding (y = 0, the cache is not touched).
template <typename T, bool kAct>
__global__ __launch_bounds__(kThreadsConv) void short_conv_step_kernel(ConvStepArgs a) {
    const int64_t c0 = ((int64_t)blockIdx.y * kThreadsConv + threadIdx.x) * 8;
    const int r = blockIdx.x;
    if (c0 >= a.C) return;
    const int s = a.slots ? a.slots[r] : r;
    const T* x = static_cast<const T*>(a.x);
    T* y = static_cast<T*>(a.y);
    float h0[8], h1[8], h2[8], xt[8], out[8];
    if (s < 0 || s >= a.n_slots) {   // padding row: y = 0, no cache access
#pragma unroll
        for (int i = 0; i < 8; ++i) out[i] = 0.f;
        Vec8<T>::store(y + (int64_t)r * a.C + c0, out);
        return;
    }
    float* st = a.cache + (int64_t)s * 3 * a.C + c0;
    load_state8(st, h0);
    load_state8(st + a.C, h1);
    load_state8(st + 2 * (int64_t)a.C, h2);
    Vec8<T>::load(x + (int64_t)r * a.C + c0, xt);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 wi = reinterpret_cast<const float4*>(a.w)[c0 + i];
        out[i] = activate<kAct>(fmaf(wi.w, xt[i], fmaf(wi.z, h2[i], fmaf(wi.y, h1[i], wi.x * h0[i]))));
    }
    Vec8<T>::store(y + (int64_t)r * a.C + c0, out);
    Vec8<float>::store(st, h1);
    Vec8<float>::store(st + a.C, h2);
    Vec8<float>::store(st + 2 * (int64_t)a.C, xt);
}

// ---------------------------------------------------------------------------
// Backward. For the loss sum <dy, y> + sum <d_final, final state>, per
// sequence and channel, with p[u] the pre-activation of token u and
// dp[u] = dy[u] act'(p[u]):
//   dx[t] = sum_i w[i] dp[t + 3 - i]   (over t + 3 - i inside the sequence)
//           + d_final[t - (eos - 3)]   (for the window's last three inputs)
//   dw[i] = sum_t dp[t] x[t - 3 + i],  d_state[j] = sum_{i <= j} w[i] dp[bos + j - i]
// A lane owns kBwdCh channels; a wave walks kBwdWaveRows consecutive tokens
// once, carrying the last three inputs of the window and the last three dp
// values: at token u it forms dp[u], adds its share of dw (u inside the
// wave's range) and completes dx[u - 3], which needs dp[u - 3 .. u]. Where a
// sequence ends, the pending dx of its last three tokens are completed with
// the terms that stay inside it, plus d_final. Tokens go in groups of up to
// kBwdGroup with every load of the group issued first; the wave's token
// range, the sequence bounds and so every branch are uniform across the wave.
// The four waves of a workgroup take consecutive token ranges of the same
// channels and sum their dw in LDS, in a fixed order, into one partial per
// workgroup; the partials are summed over workgroups by
// short_conv_bwd_finish_kernel.

// Tiling measured at T=4096, C=12288 (bf16 x, fp32 dy): 4 channels per lane,
// 64 tokens per wave and load groups of 4 tokens beat 8 channels per lane
// (more VGPRs, fewer resident waves), shorter or longer token ranges and
// groups of 2 or 8.
constexpr int kBwdCh = 4;                           // channels per lane
constexpr int kBwdWaveRows = 64;                    // tokens per wave
constexpr int kBwdWaves = 4;
constexpr int kBwdBlockRows = kBwdWaveRows * kBwdWaves;
constexpr int kBwdBlockCh = 64 * kBwdCh;            // channels per workgroup
constexpr int kBwdGroup = 4;                        // tokens whose loads are issued together

template <bool kAct>
__device__ __forceinline__ float activate_slope(float p) {
    if constexpr (kAct) {
        const float s = __builtin_amdgcn_rcpf(1.f + __expf(-p));
        return s + p * s * (1.f - s);
    }
    return 1.f;
}

struct ConvBwdLane {
    float w[kBwdCh][4];
    float dw[kBwdCh][4];
    float h0[kBwdCh], h1[kBwdCh], h2[kBwdCh];   // x[u - 3], x[u - 2], x[u - 1] of the current sequence
    float d1[kBwdCh], d2[kBwdCh], d3[kBwdCh];   // dp[u - 1], dp[u - 2], dp[u - 3]
};

// G consecutive tokens u .. u + G - 1, all inside [bos, eos): loads first,
// then dp, dw (tokens below te) and dx[t] for t = u + j - 3 in [lo, te).
template <typename T, bool kAct, int G>
__device__ __forceinline__ void conv_bwd_group(const ConvBwdArgs& a, const T* x, int64_t c0, int64_t u,
                                               int64_t lo, int64_t te, ConvBwdLane& s) {
    float xu[G][kBwdCh], dyu[G][kBwdCh];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        LoadN<T, kBwdCh>::load(x + (u + j) * a.C + c0, xu[j]);
        LoadN<float, kBwdCh>::load(a.dy + (u + j) * a.C + c0, dyu[j]);
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
        float dp[kBwdCh];
#pragma unroll
        for (int i = 0; i < kBwdCh; ++i) {
            const float p = fmaf(s.w[i][3], xu[j][i], fmaf(s.w[i][2], s.h2[i], fmaf(s.w[i][1], s.h1[i],
                                                                                  s.w[i][0] * s.h0[i])));
            dp[i] = dyu[j][i] * activate_slope<kAct>(p);
        }
        if (u + j < te) {
#pragma unroll
            for (int i = 0; i < kBwdCh; ++i) {
                s.dw[i][0] = fmaf(dp[i], s.h0[i], s.dw[i][0]);
                s.dw[i][1] = fmaf(dp[i], s.h1[i], s.dw[i][1]);
                s.dw[i][2] = fmaf(dp[i], s.h2[i], s.dw[i][2]);
                s.dw[i][3] = fmaf(dp[i], xu[j][i], s.dw[i][3]);
            }
        }
        const int64_t t = u + j - 3;
        if (t >= lo && t < te) {
            float out[kBwdCh];
#pragma unroll
            for (int i = 0; i < kBwdCh; ++i)
                out[i] = fmaf(s.w[i][0], dp[i], fmaf(s.w[i][1], s.d1[i], fmaf(s.w[i][2], s.d2[i], s.w[i][3] * s.d3[i])));
            LoadN<float, kBwdCh>::store_nt(a.dx + t * a.C + c0, out);
        }
#pragma unroll
        for (int i = 0; i < kBwdCh; ++i) {
            s.h0[i] = s.h1[i]; s.h1[i] = s.h2[i]; s.h2[i] = xu[j][i];
            s.d3[i] = s.d2[i]; s.d2[i] = s.d1[i]; s.d1[i] = dp[i];
        }
    }
}

template <typename T, bool kAct>
__global__ __launch_bounds__(64 * kBwdWaves) void short_conv_bwd_kernel(ConvBwdArgs a) {
    __shared__ float red[kBwdWaves][kBwdBlockCh * 4];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t cbase = (int64_t)blockIdx.y * kBwdBlockCh;
    const int64_t c0 = cbase + (int64_t)lane * kBwdCh;
    const int64_t BT = (int64_t)a.B * a.T;
    const int64_t tb = (int64_t)blockIdx.x * kBwdBlockRows + (int64_t)wv * kBwdWaveRows;
    const int64_t te = tb + kBwdWaveRows < BT ? tb + kBwdWaveRows : BT;
    const ConvArgs& f = a.fwd;
    const T* x = static_cast<const T*>(f.x);
    ConvBwdLane s;
#pragma unroll
    for (int i = 0; i < kBwdCh; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) s.dw[i][j] = 0.f;
    if (c0 < a.C && tb < BT) {
#pragma unroll
        for (int i = 0; i < kBwdCh; ++i) {
            const float4 wi = reinterpret_cast<const float4*>(f.w)[c0 + i];
            s.w[i][0] = wi.x; s.w[i][1] = wi.y; s.w[i][2] = wi.z; s.w[i][3] = wi.w;
            s.d1[i] = s.d2[i] = s.d3[i] = 0.f;
        }
        int n;
        int64_t bos, eos;
        find_sequence(f, tb, n, bos, eos);
        window_input_n<T, kBwdCh>(f, x, n, bos, tb - bos - 3, c0, s.h0);
        window_input_n<T, kBwdCh>(f, x, n, bos, tb - bos - 2, c0, s.h1);
        window_input_n<T, kBwdCh>(f, x, n, bos, tb - bos - 1, c0, s.h2);
        int64_t u = tb;
        for (;;) {
            if (u == eos) {
                // complete dx of the sequence's last three tokens (those in [max(tb, bos), te))
                const int64_t lo = tb > bos ? tb : bos;
#pragma unroll
                for (int r = 0; r < 3; ++r) {
                    const int64_t t = eos - 3 + r;
                    if (t < lo || t >= te) continue;
                    float out[kBwdCh];
#pragma unroll
                    for (int i = 0; i < kBwdCh; ++i) {
                        // dp[eos - 1] = d1, dp[eos - 2] = d2, dp[eos - 3] = d3
                        float acc = 0.f;
                        if (r == 0) acc = fmaf(s.w[i][1], s.d1[i], fmaf(s.w[i][2], s.d2[i], s.w[i][3] * s.d3[i]));
                        if (r == 1) acc = fmaf(s.w[i][2], s.d1[i], s.w[i][3] * s.d2[i]);
                        if (r == 2) acc = s.w[i][3] * s.d1[i];
                        out[i] = acc;
                    }
                    if (a.d_final) {
                        float df[kBwdCh];
                        LoadN<float, kBwdCh>::load(a.d_final + ((int64_t)n * 3 + r) * a.C + c0, df);
#pragma unroll
                        for (int i = 0; i < kBwdCh; ++i) out[i] += df[i];
                    }
                    LoadN<float, kBwdCh>::store_nt(a.dx + t * a.C + c0, out);
                }
                if (u >= te) break;
                find_sequence(f, u, n, bos, eos);    // the next non-empty sequence starts at u
                window_input_n<T, kBwdCh>(f, x, n, bos, -3, c0, s.h0);
                window_input_n<T, kBwdCh>(f, x, n, bos, -2, c0, s.h1);
                window_input_n<T, kBwdCh>(f, x, n, bos, -1, c0, s.h2);
#pragma unroll
                for (int i = 0; i < kBwdCh; ++i) s.d1[i] = s.d2[i] = s.d3[i] = 0.f;
            }
            const int64_t stop = eos < te + 3 ? eos : te + 3;   // dx[te - 1] needs dp up to te + 2
            if (u >= stop) break;
            const int64_t lo = tb > bos ? tb : bos;
            const int64_t rem = stop - u;
            if (rem >= kBwdGroup) {
                conv_bwd_group<T, kAct, kBwdGroup>(a, x, c0, u, lo, te, s);
                u += kBwdGroup;
            } else if (rem == 3) {
                conv_bwd_group<T, kAct, 3>(a, x, c0, u, lo, te, s);
                u += 3;
            } else if (rem == 2) {
                conv_bwd_group<T, kAct, 2>(a, x, c0, u, lo, te, s);
                u += 2;
            } else {
                conv_bwd_group<T, kAct, 1>(a, x, c0, u, lo, te, s);
                u += 1;
            }
        }
    }
    // dw of the four token ranges, summed in wave order
    float* mine = &red[wv][lane * kBwdCh * 4];
#pragma unroll
    for (int i = 0; i < kBwdCh; ++i)
        reinterpret_cast<float4*>(mine)[i] = float4{s.dw[i][0], s.dw[i][1], s.dw[i][2], s.dw[i][3]};
    __syncthreads();
    constexpr int kPer = kBwdCh;                   // floats per thread: kBwdCh / 4 channels x 4 taps
    const int e = threadIdx.x * kPer;              // (channel - cbase) * 4 + tap
    if (cbase + e / 4 < a.C) {
        float acc[kPer];
#pragma unroll
        for (int k = 0; k < kPer; ++k) acc[k] = red[0][e + k];
#pragma unroll
        for (int w2 = 1; w2 < kBwdWaves; ++w2)
#pragma unroll
            for (int k = 0; k < kPer; ++k) acc[k] += red[w2][e + k];
        LoadN<float, kPer>::store(a.part + ((int64_t)blockIdx.x * a.C + cbase) * 4 + e, acc);
    }
}

// dw[c][i] = sum over token blocks of the partials, in a fixed order.
__device__ __forceinline__ void conv_bwd_reduce(const ConvBwdArgs& a, int64_t e, int nblk) {
    if (e >= (int64_t)a.C * 4) return;    // e = c * 4 + i
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    int b = 0;
    for (; b + 4 <= nblk; b += 4)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] += a.part[(int64_t)(b + u) * a.C * 4 + e];
    for (; b < nblk; ++b) acc[0] += a.part[(int64_t)b * a.C * 4 + e];
    a.dw[e] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// Gradient of the initial conv state, one thread per (sequence, 8 channels):
// d_state[j] = sum_{i <= j} w[i] dp[bos + j - i] (tokens inside the
// sequence), plus the final-state cotangent of window entries that are still
// state entries (sequences shorter than three tokens).
template <typename T, bool kAct>
__device__ __forceinline__ void conv_bwd_dstate(const ConvBwdArgs& a, int n, int64_t c0) {
    if (c0 >= a.C) return;
    const ConvArgs& f = a.fwd;
    const T* x = static_cast<const T*>(f.x);
    int64_t bos, eos;
    if (f.cu) {
        bos = f.cu[n];
        eos = f.cu[n + 1];
    } else {
        bos = (int64_t)n * f.T;
        eos = bos + f.T;
    }
    const int64_t L = eos - bos;
    float w[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 wi = reinterpret_cast<const float4*>(f.w)[c0 + i];
        w[i][0] = wi.x; w[i][1] = wi.y; w[i][2] = wi.z; w[i][3] = wi.w;
    }
    float h0[8], h1[8], h2[8], dp[3][8];
    window_input_n<T, 8>(f, x, n, bos, -3, c0, h0);
    window_input_n<T, 8>(f, x, n, bos, -2, c0, h1);
    window_input_n<T, 8>(f, x, n, bos, -1, c0, h2);
#pragma unroll
    for (int r = 0; r < 3; ++r) {
        float xu[8], dyu[8];
        if (r < L) {
            Vec8<T>::load(x + (bos + r) * a.C + c0, xu);
            Vec8<float>::load(a.dy + (bos + r) * a.C + c0, dyu);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) xu[i] = dyu[i] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = fmaf(w[i][3], xu[i], fmaf(w[i][2], h2[i], fmaf(w[i][1], h1[i], w[i][0] * h0[i])));
            dp[r][i] = dyu[i] * activate_slope<kAct>(p);
            h0[i] = h1[i];
            h1[i] = h2[i];
            h2[i] = xu[i];
        }
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        float out[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float acc = 0.f;
#pragma unroll
            for (int k = 0; k <= j; ++k) acc += w[i][k] * dp[j - k][i];
            out[i] = acc;
        }
        // window entry L - 3 + jj is state entry j when L + jj == j
        if (a.d_final && j - L >= 0) {
            float df[8];
            Vec8<float>::load(a.d_final + ((int64_t)n * 3 + (j - L)) * a.C + c0, df);
#pragma unroll
            for (int i = 0; i < 8; ++i) out[i] += df[i];
        }
        Vec8<float>::store(a.d_state + ((int64_t)n * 3 + j) * a.C + c0, out);
    }
}

// One launch after the main pass: the first nred workgroups sum the dw
// partials, the rest take (sequence, channel group) pairs of d_state.
template <typename T, bool kAct>
__global__ __launch_bounds__(kThreadsConv) void short_conv_bwd_finish_kernel(ConvBwdArgs a, int nblk, int nred,
                                                                            int cgroups) {
    const int b = blockIdx.x;
    if (b < nred) {
        conv_bwd_reduce(a, (int64_t)b * kThreadsConv + threadIdx.x, nblk);
        return;
    }
    const int q = b - nred;
    conv_bwd_dstate<T, kAct>(a, q / cgroups, ((int64_t)(q % cgroups) * kThreadsConv + threadIdx.x) * 8);
}

template <typename T>
hipError_t launch_conv_bwd_t(const ConvBwdArgs& a, hipStream_t s) {
    const int64_t BT = (int64_t)a.B * a.T;
    const unsigned cgroups = (unsigned)((a.C / 8 + kThreadsConv - 1) / kThreadsConv);
    const int64_t nblk = (BT + kBwdBlockRows - 1) / kBwdBlockRows;
    if (nblk > 0) {
        const dim3 grid((unsigned)nblk, (unsigned)((a.C + kBwdBlockCh - 1) / kBwdBlockCh));
        if (a.fwd.act)
            hipLaunchKernelGGL((short_conv_bwd_kernel<T, true>), grid, dim3(64 * kBwdWaves), 0, s, a);
        else
            hipLaunchKernelGGL((short_conv_bwd_kernel<T, false>), grid, dim3(64 * kBwdWaves), 0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int nred = (int)((a.C * 4 + kThreadsConv - 1) / kThreadsConv);
    const int64_t nstate = a.d_state ? (int64_t)a.N * cgroups : 0;
    if (nred + nstate > (int64_t)0x7fffffff) return hipErrorInvalidValue;
    const dim3 fgrid((unsigned)(nred + nstate));
    if (a.fwd.act)
        hipLaunchKernelGGL((short_conv_bwd_finish_kernel<T, true>), fgrid, dim3(kThreadsConv), 0, s, a, (int)nblk,
                           nred, (int)cgroups);
    else
        hipLaunchKernelGGL((short_conv_bwd_finish_kernel<T, false>), fgrid, dim3(kThreadsConv), 0, s, a, (int)nblk,
                           nred, (int)cgroups);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_conv_t(const ConvArgs* a, int count, hipStream_t s) {
    ConvSet set;
    int64_t cmax = 0;
    bool any_y = false, any_state = false;
    for (int i = 0; i < count; ++i) {
        set.p[i] = a[i];
        cmax = std::max<int64_t>(cmax, a[i].C);
        any_y |= a[i].y != nullptr;            // (a null y: only the final state)
        any_state |= a[i].state_out != nullptr;
    }
    const int64_t BT = (int64_t)a[0].B * a[0].T;
    if (BT > 0 && any_y) {
        const dim3 grid((unsigned)((BT + kFwdBlockRows - 1) / kFwdBlockRows),
                        (unsigned)((cmax + kFwdBlockCh - 1) / kFwdBlockCh), (unsigned)count);
        if (a[0].act)
            hipLaunchKernelGGL((short_conv_kernel<T, true>), grid, dim3(256), 0, s, set);
        else
            hipLaunchKernelGGL((short_conv_kernel<T, false>), grid, dim3(256), 0, s, set);
    }
    if (any_state && a[0].N > 0) {
        const unsigned cgroups = (unsigned)((cmax / 8 + kThreadsConv - 1) / kThreadsConv);
        hipLaunchKernelGGL((short_conv_state_kernel<T>), dim3((unsigned)a[0].N, cgroups, (unsigned)count),
                           dim3(kThreadsConv), 0, s, set);
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_conv_step_t(const ConvStepArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)a.Nb, (unsigned)((a.C / 8 + kThreadsConv - 1) / kThreadsConv));
    if (a.act)
        hipLaunchKernelGGL((short_conv_step_kernel<T, true>), grid, dim3(kThreadsConv), 0, s, a);
    else
        hipLaunchKernelGGL((short_conv_step_kernel<T, false>), grid, dim3(kThreadsConv), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_short_conv(const ConvArgs& a, hipStream_t s) {
    return launch_short_conv_set(&a, 1, s);
}

hipError_t launch_short_conv_set(const ConvArgs* a, int count, hipStream_t s) {
    if (count < 1 || count > kMaxConvSet) return hipErrorInvalidValue;
    return a[0].bf16 ? launch_conv_t<__bf16>(a, count, s) : launch_conv_t<float>(a, count, s);
}

hipError_t launch_short_conv_step(const ConvStepArgs& a, hipStream_t s) {
    return a.bf16 ? launch_conv_step_t<__bf16>(a, s) : launch_conv_step_t<float>(a, s);
}

int64_t short_conv_bwd_blocks(int32_t B, int32_t T) {
    return ((int64_t)B * T + kBwdBlockRows - 1) / kBwdBlockRows;
}

hipError_t launch_short_conv_bwd(const ConvBwdArgs& a, hipStream_t s) {
    return a.fwd.bf16 ? launch_conv_bwd_t<__bf16>(a, s) : launch_conv_bwd_t<float>(a, s);
}

}  // namespace kda
