// Backward through the gate, beta and L2-norm prologue of the chunk forward.
//
// The prologue, per token t and head h (channel c):
//   q = x_q / n_q, n_q = sqrt(|x_q|^2 + eps)           (k likewise)
//   g = lb * s, s = sigmoid(z), z = e^{A_log[c]} (x_g + dt_bias[h, c])
//   beta = sigmoid(y)
// One call of the backward from raw projections:
//   1. prologue_apply_kernel: q, k, g, beta (and v, dO widened) in float32;
//   2. the recurrence's backward on those (launch_chunk_bwd), which writes dq,
//      dk, dg, dbeta into the caller's gradient buffers;
//   3. prologue_grad_kernel: in place, dx_q = dq / n_q - x_q (x_q . dq) / n_q^3
//      (k likewise), dz = dg lb s (1 - s), dx_g = dz e^{A_log}, dy = dbeta beta
//      (1 - beta); and per (token block, head, channel) partial sums of
//      dz e^{A_log} (for dt_bias) and dz z (for A_log);
//   4. prologue_reduce_kernel: those partials summed in a fixed order.
#include "device_common.hpp"
#include "launchers.hpp"

namespace kda {
namespace {

constexpr int kTokBlock = 64;   // tokens per workgroup of the prologue kernels

// Sum over the workgroup's channel threads (blockDim.x = max(DK, 64), one or
// two waves); every thread gets the totals. `red` holds 2 waves x NV floats.
template <int NV>
__device__ __forceinline__ void block_sum(float (&v)[NV], float* red) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) v[i] += __shfl_xor(v[i], m, 64);
    if (blockDim.x > 64) {
        const int w = threadIdx.x >> 6;
        __syncthreads();
        if ((threadIdx.x & 63) == 0)
#pragma unroll
            for (int i = 0; i < NV; ++i) red[w * NV + i] = v[i];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] = red[i] + red[NV + i];
    }
}

__device__ __forceinline__ float sigmoid(float z) { return 1.f / (1.f + __expf(-z)); }

template <typename Tin, int DK>
__global__ __launch_bounds__(128) void prologue_apply_kernel(PrologueBwdArgs a) {
    __shared__ float red[2 * 2];
    const int c = threadIdx.x;
    const bool on = c < DK;
    const int h = blockIdx.y;
    const int64_t rows_total = (int64_t)a.B * a.T;
    const float eA = on ? __expf(a.A_log[c]) : 0.f;
    const float bias = on ? a.dt_bias[h * DK + c] : 0.f;
    const Tin* xq = static_cast<const Tin*>(a.q_raw);
    const Tin* xk = static_cast<const Tin*>(a.k_raw);
    const Tin* xg = static_cast<const Tin*>(a.g_logit);
    const Tin* xb = static_cast<const Tin*>(a.beta_logit);
    const Tin* v = static_cast<const Tin*>(a.v);
    const Tin* d_o = static_cast<const Tin*>(a.d_o);
    const int64_t t_end = min((int64_t)(blockIdx.x + 1) * kTokBlock, rows_total);
    for (int64_t t = (int64_t)blockIdx.x * kTokBlock; t < t_end; ++t) {
        const int64_t row = t * a.H + h;
        const float q = on ? load_elem(xq, row * DK + c) : 0.f;
        const float k = on ? load_elem(xk, row * DK + c) : 0.f;
        float s[2] = {q * q, k * k};
        block_sum(s, red);
        if (on) {
            a.qf[row * DK + c] = q / sqrtf(s[0] + a.l2_eps);
            a.kf[row * DK + c] = k / sqrtf(s[1] + a.l2_eps);
            a.gf[row * DK + c] = a.gate_lb * sigmoid(eA * (load_elem(xg, row * DK + c) + bias));
        }
        if (c == 0) a.bf[row] = sigmoid(load_elem(xb, row));
        for (int j = c; j < a.Dv; j += blockDim.x) {
            a.vf[row * a.Dv + j] = load_elem(v, row * a.Dv + j);
            a.dof[row * a.Dv + j] = load_elem(d_o, row * a.Dv + j);
        }
    }
}

template <typename Tin, int DK>
__global__ __launch_bounds__(128) void prologue_grad_kernel(PrologueBwdArgs a) {
    __shared__ float red[2 * 4];
    const int c = threadIdx.x;
    const bool on = c < DK;
    const int h = blockIdx.y;
    const int64_t rows_total = (int64_t)a.B * a.T;
    const float eA = on ? __expf(a.A_log[c]) : 0.f;
    const float bias = on ? a.dt_bias[h * DK + c] : 0.f;
    const Tin* xq = static_cast<const Tin*>(a.q_raw);
    const Tin* xk = static_cast<const Tin*>(a.k_raw);
    const Tin* xg = static_cast<const Tin*>(a.g_logit);
    const Tin* xb = static_cast<const Tin*>(a.beta_logit);
    float acc_b = 0.f, acc_A = 0.f;
    const int64_t t_end = min((int64_t)(blockIdx.x + 1) * kTokBlock, rows_total);
    for (int64_t t = (int64_t)blockIdx.x * kTokBlock; t < t_end; ++t) {
        const int64_t row = t * a.H + h;
        const int64_t e = row * DK + c;
        const float q = on ? load_elem(xq, e) : 0.f;
        const float k = on ? load_elem(xk, e) : 0.f;
        const float dq = on ? a.dq[e] : 0.f;
        const float dk = on ? a.dk[e] : 0.f;
        float s[4] = {q * q, q * dq, k * k, k * dk};
        block_sum(s, red);
        if (on) {
            const float nq = sqrtf(s[0] + a.l2_eps), nk = sqrtf(s[2] + a.l2_eps);
            a.dq[e] = dq / nq - q * s[1] / (nq * nq * nq);
            a.dk[e] = dk / nk - k * s[3] / (nk * nk * nk);
            const float z = eA * (load_elem(xg, e) + bias);
            const float sg = sigmoid(z);
            const float dz = a.dg[e] * a.gate_lb * sg * (1.f - sg);
            a.dg[e] = dz * eA;
            acc_b += dz * eA;
            acc_A += dz * z;
        }
        if (c == 0) {
            const float sb = sigmoid(load_elem(xb, row));
            a.dbeta[row] = a.dbeta[row] * sb * (1.f - sb);
        }
    }
    if (on) {
        const int64_t p = ((int64_t)blockIdx.x * a.H + h) * DK + c;
        a.part_b[p] = acc_b;
        a.part_A[p] = acc_A;
    }
}

// ddt_bias[h][c] = sum over token blocks; dA_log[c] = sum over token blocks and
// heads; one thread per output, in a fixed order.
__global__ void prologue_reduce_kernel(PrologueBwdArgs a, int nblk, int DK) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    const int n_bias = a.H * DK;
    if (i < n_bias) {
        const int h = i / DK, c = i % DK;
        float acc = 0.f;
        for (int b = 0; b < nblk; ++b) acc += a.part_b[((int64_t)b * a.H + h) * DK + c];
        a.d_dt_bias[i] = acc;
    } else if (i < n_bias + DK) {
        const int c = i - n_bias;
        float acc = 0.f;
        for (int b = 0; b < nblk; ++b)
            for (int h = 0; h < a.H; ++h) acc += a.part_A[((int64_t)b * a.H + h) * DK + c];
        a.d_A_log[c] = acc;
    }
}

template <typename Tin>
hipError_t launch_apply(const PrologueBwdArgs& a, dim3 grid, hipStream_t s, bool grad) {
    const dim3 block(a.Dk > 64 ? a.Dk : 64);
    switch (a.Dk) {
        case 16:
            if (grad) prologue_grad_kernel<Tin, 16><<<grid, block, 0, s>>>(a);
            else prologue_apply_kernel<Tin, 16><<<grid, block, 0, s>>>(a);
            break;
        case 32:
            if (grad) prologue_grad_kernel<Tin, 32><<<grid, block, 0, s>>>(a);
            else prologue_apply_kernel<Tin, 32><<<grid, block, 0, s>>>(a);
            break;
        case 64:
            if (grad) prologue_grad_kernel<Tin, 64><<<grid, block, 0, s>>>(a);
            else prologue_apply_kernel<Tin, 64><<<grid, block, 0, s>>>(a);
            break;
        default:
            if (grad) prologue_grad_kernel<Tin, 128><<<grid, block, 0, s>>>(a);
            else prologue_apply_kernel<Tin, 128><<<grid, block, 0, s>>>(a);
            break;
    }
    return hipGetLastError();
}

}  // namespace

int64_t prologue_bwd_token_blocks(int32_t B, int32_t T) {
    return ((int64_t)B * T + kTokBlock - 1) / kTokBlock;
}

hipError_t launch_prologue_bwd(const PrologueBwdArgs& p, const BwdArgs& core, hipStream_t s) {
    const int64_t nblk = prologue_bwd_token_blocks(p.B, p.T);
    hipError_t e;
    if (nblk > 0) {
        const dim3 grid((unsigned)nblk, (unsigned)p.H);
        e = p.bf16 ? launch_apply<__bf16>(p, grid, s, false) : launch_apply<float>(p, grid, s, false);
        if (e != hipSuccess) return e;
    }
    if ((e = launch_chunk_bwd(core, s)) != hipSuccess) return e;
    if (nblk > 0) {
        const dim3 grid((unsigned)nblk, (unsigned)p.H);
        e = p.bf16 ? launch_apply<__bf16>(p, grid, s, true) : launch_apply<float>(p, grid, s, true);
        if (e != hipSuccess) return e;
        const int n_out = p.H * p.Dk + p.Dk;
        prologue_reduce_kernel<<<dim3((unsigned)((n_out + 255) / 256)), dim3(256), 0, s>>>(p, (int)nblk, p.Dk);
        return hipGetLastError();
    }
    // no tokens: the reduction over zero token blocks writes zeros
    const int n_out = p.H * p.Dk + p.Dk;
    prologue_reduce_kernel<<<dim3((unsigned)((n_out + 255) / 256)), dim3(256), 0, s>>>(p, 0, p.Dk);
    return hipGetLastError();
}

PrologueBwdLayout prologue_bwd_layout(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t N,
                                      bool packed) {
    auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
    const int64_t rows = (int64_t)B * T * H;
    const int64_t nblk = prologue_bwd_token_blocks(B, T);
    PrologueBwdLayout L;
    int64_t off = 0;
    L.core = off;  off += up(chunk_bwd_ws_floats(B, T, H, Dk, Dv, N, packed) * 4);
    L.qf = off;    off += up(rows * Dk * 4);
    L.kf = off;    off += up(rows * Dk * 4);
    L.gf = off;    off += up(rows * Dk * 4);
    L.bf = off;    off += up(rows * 4);
    L.vf = off;    off += up(rows * Dv * 4);
    L.dof = off;   off += up(rows * Dv * 4);
    L.part_b = off; off += up(nblk * H * Dk * 4);
    L.part_A = off; off += up(nblk * H * Dk * 4);
    L.bytes = off;
    return L;
}

}  // namespace kda
