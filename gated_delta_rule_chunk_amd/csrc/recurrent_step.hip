// KDA decode step (one token per row) against a float32 state cache, in place.
//
// One workgroup per (row, head) streams that head's d_k x d_v float32 state
// once from HBM and once back:
//   S' = Diag(exp g) S;  x = S'^T k;  y = S'^T q;  u = beta (v - x)
//   o  = scale * (y + (k.q) u)            (= scale * S_new^T q)
//   S  = S' + k u^T
// The state is the only large operand (64 KiB per head at d=128), so the
// kernel is bound by HBM bandwidth: each thread keeps its slice of S' in
// registers between the two reductions and the write-back, and every state
// access is a coalesced 16-byte load or store along d_v. State loads and
// stores are non-temporal: each byte is read and written once per step, and
// the hint keeps the stream from displacing other lines in the caches (7%
// faster than plain accesses at 256 rows x 96 heads).
//
// From raw projections (kIn >= 1) the same workgroup first forms the token's
// inputs while its state loads are in flight, as the chunk forward's prologue
// does: q and k scaled to unit length, g = lb sigmoid(exp(A_log) (logit +
// dt_bias)), beta = sigmoid(logit); with kIn = 2 the short-convolution step of
// q, k and v comes before that, in the same fma order and with the same
// rounding of its output to the input type as the standalone convolution
// step, its cache shifted in place. Wave 0 takes q and k (two channels per
// lane, and the three sums |q|^2, |k|^2, k.q by a butterfly), wave 1 the
// gate, waves 2 and 3 v; the state update after the first barrier is the
// plain step's.
//
// A row whose slot lies outside [0, n_slots) (e.g. -1 for a padding row of a
// serving batch) touches no state and no convolution cache: its output is
// zero.
#include "device_common.hpp"
#include "launchers.hpp"

namespace kda {
namespace {

// Threads per workgroup: four float4 state elements per thread for the large
// heads. At 128 x 128 (1024 threads) the step runs at the rate of a plain
// in-place read-modify-write stream of the same bytes; 256 threads with 16
// float4 each were 6% slower, 512 with 8 each 3%.
template <int DK, int DV> constexpr int step_threads() {
    return DK * DV >= 16384 ? 1024 : DK * DV >= 8192 ? 512 : 256;
}

// Sum of v over lanes l and l ^ M of the wave (the same value on both lanes).
template <int M> __device__ __forceinline__ float fold_lane(float v) {
    if constexpr (M == 32) {
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        return __uint_as_float(p[0]) + __uint_as_float(p[1]);
    } else if constexpr (M == 16) {
        const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        return __uint_as_float(p[0]) + __uint_as_float(p[1]);
    } else {
        return v + __shfl_xor(v, M);
    }
}
// Sum of v over the lanes of the wave that share lane % M0 (fold_rows<M0>).
template <int M> __device__ __forceinline__ f32x4 fold_rows(f32x4 v) {
    if constexpr (M >= 64) {
        return v;
    } else {
        v = f32x4{fold_lane<M>(v.x), fold_lane<M>(v.y), fold_lane<M>(v.z), fold_lane<M>(v.w)};
        return fold_rows<M * 2>(v);
    }
}

template <typename T> __device__ __forceinline__ float round_to(float x);
template <> __device__ __forceinline__ float round_to<float>(float x) { return x; }
template <> __device__ __forceinline__ float round_to<__bf16>(float x) { return bf16_bits_to_f32(f32_to_bf16_bits(x)); }

// Channel c of projection j (0 q, 1 k, 2 v; D channels per head) for token
// tok: the loaded value, or with kConv the convolution step over the cache of
// the row's slot (window h0, h1, h2, x oldest first), which it shifts.
template <typename Tin, bool kConv>
__device__ __forceinline__ float raw_input(const StepArgs& a, int j, const Tin* x, int64_t tok, int D, int h,
                                           int slot, int c) {
    const float xv = load_elem(x, tok * D + c);
    if constexpr (!kConv) {
        return xv;
    } else {
        const int64_t C = (int64_t)a.H * D;
        float* st = a.conv_cache[j] + (int64_t)slot * 3 * C + (int64_t)h * D + c;
        const float h0 = st[0], h1 = st[C], h2 = st[2 * C];
        const float4 w = reinterpret_cast<const float4*>(a.conv_w[j])[(int64_t)h * D + c];
        float y = fmaf(w.w, xv, fmaf(w.z, h2, fmaf(w.y, h1, w.x * h0)));
        if (a.conv_act) y = y * __builtin_amdgcn_rcpf(1.f + __expf(-y));
        st[0] = h1;
        st[C] = h2;
        st[2 * C] = xv;
        return round_to<Tin>(y);
    }
}

// kIn: 0 prepared inputs, 1 raw projections, 2 convolution inputs. At most
// 128 VGPRs (four waves per SIMD) in every variant.
template <int DK, int DV, typename Tin, int kIn>
__global__ __launch_bounds__((step_threads<DK, DV>())) __attribute__((amdgpu_waves_per_eu(4))) void
recurrent_step_kernel(StepArgs a) {
    constexpr int kStepThreads = step_threads<DK, DV>();
    constexpr int QUADS = DV / 4;                 // float4 columns per row
    constexpr int RG = kStepThreads / QUADS;      // row groups
    constexpr int ROWS = (DK + RG - 1) / RG;      // rows per thread
    constexpr int W = kStepThreads / 64;          // waves
    __shared__ float sk[DK], sq[DK], seg[DK], sv[DV];
    __shared__ f32x4 redx[W][QUADS];
    __shared__ f32x4 redy[W][QUADS];
    __shared__ float skq;
    __shared__ f32x4 su[QUADS];

    const Tin* q = static_cast<const Tin*>(a.q);
    const Tin* k = static_cast<const Tin*>(a.k);
    const Tin* v = static_cast<const Tin*>(a.v);
    const Tin* g = static_cast<const Tin*>(a.g);
    const Tin* beta = static_cast<const Tin*>(a.beta);
    Tin* o = static_cast<Tin*>(a.o);

    const int tid = threadIdx.x;
    const int row = blockIdx.x / a.H;
    const int h = blockIdx.x % a.H;
    const int slot = a.slots ? a.slots[row] : row;
    const int64_t tok = (int64_t)row * a.H + h;
    if (slot < 0 || slot >= a.n_slots) {   // padding row (uniform over the workgroup)
        for (int i = tid; i < DV; i += kStepThreads) store_elem(o, tok * DV + i, 0.f);
        return;
    }
    f32x4* S = reinterpret_cast<f32x4*>(a.cache + ((int64_t)slot * a.H + h) * DK * DV);

    const int quad = tid % QUADS;
    const int rg = tid / QUADS;

    // issue the state loads first: they are the bulk of the traffic
    f32x4 s[ROWS];
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const int r = rg + RG * i;
        s[i] = (r < DK) ? __builtin_nontemporal_load(&S[r * QUADS + quad]) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float bt;
    if constexpr (kIn == 0) {
        for (int i = tid; i < DK; i += kStepThreads) {
            sk[i] = load_elem(k, tok * DK + i);
            sq[i] = load_elem(q, tok * DK + i);
            seg[i] = expf(load_elem(g, tok * DK + i));
        }
        for (int i = tid; i < DV; i += kStepThreads) sv[i] = load_elem(v, tok * DV + i);
        if (tid < 64) {
            float p = 0.f;
            for (int i = tid; i < DK; i += 64) p += load_elem(k, tok * DK + i) * load_elem(q, tok * DK + i);
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off);
            if (tid == 0) skq = p;
        }
        bt = load_elem(beta, tok);
    } else {
        constexpr bool kConv = kIn == 2;
        if (tid < 64) {
            float qv[2], kv[2];
            float qq = 0.f, kk = 0.f, kq = 0.f;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int c = tid + 64 * i;
                qv[i] = c < DK ? raw_input<Tin, kConv>(a, 0, q, tok, DK, h, slot, c) : 0.f;
                kv[i] = c < DK ? raw_input<Tin, kConv>(a, 1, k, tok, DK, h, slot, c) : 0.f;
                qq += qv[i] * qv[i];
                kk += kv[i] * kv[i];
                kq += kv[i] * qv[i];
            }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                qq += __shfl_xor(qq, off);
                kk += __shfl_xor(kk, off);
                kq += __shfl_xor(kq, off);
            }
            // eps > 0: a row of zeros normalises to zeros
            const float rq = 1.f / sqrtf(qq + a.l2_eps), rk = 1.f / sqrtf(kk + a.l2_eps);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int c = tid + 64 * i;
                if (c < DK) {
                    sq[c] = qv[i] * rq;
                    sk[c] = kv[i] * rk;
                }
            }
            if (tid == 0) skq = kq * rq * rk;
        } else if (tid < 128) {
            for (int c = tid - 64; c < DK; c += 64) {
                const float gl = load_elem(g, tok * DK + c);
                const float gv = a.gate_lb / (1.f + expf(-expf(a.A_log[c]) * (gl + a.dt_bias[h * DK + c])));
                seg[c] = expf(gv);
            }
        } else {
            for (int c = tid - 128; c < DV; c += 128) sv[c] = raw_input<Tin, kConv>(a, 2, v, tok, DV, h, slot, c);
        }
        bt = 1.f / (1.f + expf(-load_elem(beta, tok)));
    }
    __syncthreads();

    f32x4 x = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const int r = rg + RG * i;
        if (r < DK) {
            s[i] *= seg[r];
            x += sk[r] * s[i];
            y += sq[r] * s[i];
        }
    }
    // x and y over all rows: the row groups of each wave fold by lane swaps
    // (lanes l and l ^ m for m = QUADS .. 32 share a column quad), the waves'
    // partials meet in LDS, wave 0 sums them in wave order, forms u and o, and
    // hands u back through LDS.
    x = fold_rows<QUADS>(x);
    y = fold_rows<QUADS>(y);
    const int w = tid / 64, lane = tid % 64;
    if (lane < QUADS) {
        redx[w][lane] = x;
        redy[w][lane] = y;
    }
    __syncthreads();
    if (tid < QUADS) {
        x = redx[0][tid];
        y = redy[0][tid];
#pragma unroll
        for (int j = 1; j < W; ++j) {
            x += redx[j][tid];
            y += redy[j][tid];
        }
        const f32x4 vv = {sv[4 * tid], sv[4 * tid + 1], sv[4 * tid + 2], sv[4 * tid + 3]};
        const f32x4 uq = bt * (vv - x);
        const f32x4 ov = a.scale * (y + skq * uq);
        const int64_t ob = tok * DV + 4 * tid;
        store_elem(o, ob + 0, ov.x);
        store_elem(o, ob + 1, ov.y);
        store_elem(o, ob + 2, ov.z);
        store_elem(o, ob + 3, ov.w);
        su[tid] = uq;
    }
    __syncthreads();
    const f32x4 u = su[quad];
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const int r = rg + RG * i;
        if (r < DK) __builtin_nontemporal_store(s[i] + sk[r] * u, &S[r * QUADS + quad]);
    }
}

template <int DK, int DV, typename Tin>
hipError_t launch_in(const StepArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)(a.Nb * a.H)), block(step_threads<DK, DV>());
    if (a.conv)
        hipLaunchKernelGGL((recurrent_step_kernel<DK, DV, Tin, 2>), grid, block, 0, s, a);
    else if (a.prologue)
        hipLaunchKernelGGL((recurrent_step_kernel<DK, DV, Tin, 1>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((recurrent_step_kernel<DK, DV, Tin, 0>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_dims(const StepArgs& a, hipStream_t s) {
    return a.bf16 ? launch_in<DK, DV, __bf16>(a, s) : launch_in<DK, DV, float>(a, s);
}

template <int DK>
hipError_t launch_dk(const StepArgs& a, hipStream_t s) {
    switch (a.Dv) {
        case 16: return launch_dims<DK, 16>(a, s);
        case 32: return launch_dims<DK, 32>(a, s);
        case 64: return launch_dims<DK, 64>(a, s);
        case 128: return launch_dims<DK, 128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_recurrent_step(const StepArgs& a, hipStream_t s) {
    if (a.Nb == 0) return hipSuccess;
    if (a.conv && !a.prologue) return hipErrorInvalidValue;
    switch (a.Dk) {
        case 16: return launch_dk<16>(a, s);
        case 32: return launch_dk<32>(a, s);
        case 64: return launch_dk<64>(a, s);
        case 128: return launch_dk<128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
