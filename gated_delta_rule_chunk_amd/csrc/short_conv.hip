// Short causal depthwise convolution over time (kernel 4) of the q, k or v
// projections, with a per-sequence conv state, and its decode step.
//
// Per sequence and channel c, with the window ending at token t:
//   y[t][c] = sum_{i=0..3} w[c][i] * x[t - 3 + i][c]
// where the three inputs before the sequence's first token come from the conv
// state ([N][3][C]: x[-3], x[-2], x[-1]) or are zero; with the activation,
// y <- y * sigmoid(y). The final state is the window's last three inputs.
//
// The kernels are bandwidth-bound: a thread owns 8 consecutive channels (16
// bytes of bf16) of kRows consecutive tokens and keeps the three previous
// inputs in registers, so a wave reads and writes 1 KiB contiguous per token
// and every input is read once (plus a three-token halo per kRows).
#include "device_common.hpp"
#include "launchers.hpp"

namespace kda {
namespace {

constexpr int kRows = 8;         // tokens per thread
constexpr int kThreadsConv = 256;

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

// input x[tau] of sequence n, tau relative to the sequence start (tau >= -3)
template <typename T>
__device__ __forceinline__ void window_input(const ConvArgs& a, const T* x, int n, int64_t bos, int64_t tau,
                                             int64_t c0, float (&f)[8]) {
    if (tau >= 0) {
        Vec8<T>::load(x + (bos + tau) * a.C + c0, f);
    } else if (a.state_in) {
        load_state8(a.state_in + ((int64_t)n * 3 + (3 + tau)) * a.C + c0, f);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = 0.f;
    }
}

template <typename T, bool kAct>
__global__ __launch_bounds__(kThreadsConv) void short_conv_kernel(ConvArgs a) {
    const int64_t c0 = ((int64_t)blockIdx.y * kThreadsConv + threadIdx.x) * 8;
    if (c0 >= a.C) return;
    const int64_t BT = (int64_t)a.B * a.T;
    const int64_t t0 = (int64_t)blockIdx.x * kRows;
    if (t0 >= BT) return;
    const T* x = static_cast<const T*>(a.x);
    T* y = static_cast<T*>(a.y);
    float w[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 wi = reinterpret_cast<const float4*>(a.w)[c0 + i];
        w[i][0] = wi.x; w[i][1] = wi.y; w[i][2] = wi.z; w[i][3] = wi.w;
    }
    int n;
    int64_t bos, eos;
    find_sequence(a, t0, n, bos, eos);
    if constexpr (sizeof(T) == 2) {
        if (t0 - bos >= 3 && t0 + kRows <= eos) {
            // the common case: the whole block and its halo inside one sequence.
            // All kRows + 3 rows are loaded before any is used, so the loads overlap.
            uint4 raw[kRows + 3];
#pragma unroll
            for (int r = 0; r < kRows + 3; ++r)
                raw[r] = *reinterpret_cast<const uint4*>(x + (t0 - 3 + r) * a.C + c0);
#pragma unroll
            for (int r = 0; r < kRows; ++r) {
                float f0[8], f1[8], f2[8], f3[8], out[8];
                unpack8(raw[r], f0);
                unpack8(raw[r + 1], f1);
                unpack8(raw[r + 2], f2);
                unpack8(raw[r + 3], f3);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    out[i] = activate<kAct>(fmaf(w[i][3], f3[i], fmaf(w[i][2], f2[i], fmaf(w[i][1], f1[i], w[i][0] * f0[i]))));
                Vec8<T>::store(y + (t0 + r) * a.C + c0, out);
            }
            return;
        }
    }
    float h0[8], h1[8], h2[8];      // x[t-3], x[t-2], x[t-1]
    window_input<T>(a, x, n, bos, t0 - bos - 3, c0, h0);
    window_input<T>(a, x, n, bos, t0 - bos - 2, c0, h1);
    window_input<T>(a, x, n, bos, t0 - bos - 1, c0, h2);
    const int rows = (int)((BT - t0) < kRows ? (BT - t0) : kRows);
    for (int r = 0; r < rows; ++r) {
        const int64_t t = t0 + r;
        if (t == eos) {
            // the next non-empty sequence starts here: its window starts from its state
            find_sequence(a, t, n, bos, eos);
            window_input<T>(a, x, n, bos, -3, c0, h0);
            window_input<T>(a, x, n, bos, -2, c0, h1);
            window_input<T>(a, x, n, bos, -1, c0, h2);
        }
        float xt[8], out[8];
        Vec8<T>::load(x + t * a.C + c0, xt);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float acc = fmaf(w[i][3], xt[i], fmaf(w[i][2], h2[i], fmaf(w[i][1], h1[i], w[i][0] * h0[i])));
            out[i] = activate<kAct>(acc);
            h0[i] = h1[i];
            h1[i] = h2[i];
            h2[i] = xt[i];
        }
        Vec8<T>::store(y + t * a.C + c0, out);
    }
}

// Final conv state of every sequence: its window's last three inputs. One
// thread per (sequence, 8 channels) reads all three before writing, so the
// output may alias the input state.
template <typename T>
__global__ __launch_bounds__(kThreadsConv) void short_conv_state_kernel(ConvArgs a) {
    const int64_t c0 = ((int64_t)blockIdx.y * kThreadsConv + threadIdx.x) * 8;
    const int n = blockIdx.x;
    if (c0 >= a.C) return;
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
    for (int j = 0; j < 3; ++j) window_input<T>(a, x, n, bos, L - 3 + j, c0, f[j]);
#pragma unroll
    for (int j = 0; j < 3; ++j) Vec8<float>::store(a.state_out + ((int64_t)n * 3 + j) * a.C + c0, f[j]);
}

// Decode: row r reads and shifts cache[slot(r)] ([3][C]).
template <typename T, bool kAct>
__global__ __launch_bounds__(kThreadsConv) void short_conv_step_kernel(ConvStepArgs a) {
    const int64_t c0 = ((int64_t)blockIdx.y * kThreadsConv + threadIdx.x) * 8;
    const int r = blockIdx.x;
    if (c0 >= a.C) return;
    const int s = a.slots ? a.slots[r] : r;
    float* st = a.cache + (int64_t)s * 3 * a.C + c0;
    const T* x = static_cast<const T*>(a.x);
    T* y = static_cast<T*>(a.y);
    float h0[8], h1[8], h2[8], xt[8], out[8];
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

template <typename T>
hipError_t launch_conv_t(const ConvArgs& a, hipStream_t s) {
    const int64_t BT = (int64_t)a.B * a.T;
    const unsigned cgroups = (unsigned)((a.C / 8 + kThreadsConv - 1) / kThreadsConv);
    if (BT > 0) {
        const dim3 grid((unsigned)((BT + kRows - 1) / kRows), cgroups);
        if (a.act)
            hipLaunchKernelGGL((short_conv_kernel<T, true>), grid, dim3(kThreadsConv), 0, s, a);
        else
            hipLaunchKernelGGL((short_conv_kernel<T, false>), grid, dim3(kThreadsConv), 0, s, a);
    }
    if (a.state_out && a.N > 0)
        hipLaunchKernelGGL((short_conv_state_kernel<T>), dim3((unsigned)a.N, cgroups), dim3(kThreadsConv), 0, s, a);
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
    return a.bf16 ? launch_conv_t<__bf16>(a, s) : launch_conv_t<float>(a, s);
}

hipError_t launch_short_conv_step(const ConvStepArgs& a, hipStream_t s) {
    return a.bf16 ? launch_conv_step_t<__bf16>(a, s) : launch_conv_step_t<float>(a, s);
}

}  // namespace kda
