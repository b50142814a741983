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
//   4. prologue_reduce_bias_kernel, prologue_reduce_alog_kernel: those partials
//      summed in a fixed order.
// Step 1 alone, with outputs in the input dtype, is the standalone prologue
// (kda_prologue).
#include "device_common.hpp"
#include "launchers.hpp"

namespace kda {
namespace {

constexpr int kTokBlock = 64;   // tokens per workgroup of the prologue kernels

constexpr int kPThreads = 256;

// Eight consecutive input elements (16 bytes of bf16 or 32 of float32).
template <typename T> __device__ __forceinline__ void load8(const T* p, int64_t i, float* o);
template <> __device__ __forceinline__ void load8<float>(const float* p, int64_t i, float* o) {
    const float4 a = *reinterpret_cast<const float4*>(p + i);
    const float4 b = *reinterpret_cast<const float4*>(p + i + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
template <> __device__ __forceinline__ void load8<__bf16>(const __bf16* p, int64_t i, float* o) {
    unpack8(*reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p) + i), o);
}
__device__ __forceinline__ void store8(float* p, int64_t i, const float* v) {
    *reinterpret_cast<float4*>(p + i) = float4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<float4*>(p + i + 4) = float4{v[4], v[5], v[6], v[7]};
}
__device__ __forceinline__ void store8(__bf16* p, int64_t i, const float* v) {
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p) + i) =
        uint4{pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]), pack2_bf16(v[4], v[5]), pack2_bf16(v[6], v[7])};
}

// Sum over the L lanes (a power of two, at most 16) that share a row: every
// lane of the group gets the total.
template <int L>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int m = 1; m < L; m <<= 1) v += __shfl_xor(v, m, 64);
    return v;
}

__device__ __forceinline__ float sigmoid(float z) { return 1.f / (1.f + __expf(-z)); }

// One workgroup per (block of kTokBlock tokens, head). L = DK/8 lanes hold
// one (token, head) row, eight channels each, and 256/L rows go at once; row
// sums are shuffles within the L lanes. q, k, g and beta are written as Tout
// (float32 for the backward, the input dtype for kda_prologue); each lane
// writes only the elements it has read, so an output may be its own input.
template <typename Tin, typename Tout, int DK>
__global__ __launch_bounds__(kPThreads) void prologue_apply_kernel(PrologueBwdArgs a) {
    constexpr int L = DK / 8, RPI = kPThreads / L;
    const int tid = threadIdx.x, part = tid % L, rg = tid / L, c0 = 8 * part;
    const int h = blockIdx.y;
    const int64_t rows_total = (int64_t)a.B * a.T;
    const int64_t t0 = (int64_t)blockIdx.x * kTokBlock;
    const int64_t t_end = min(t0 + kTokBlock, rows_total);
    float eA[8], bias[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        eA[u] = __expf(a.A_log[c0 + u]);
        bias[u] = a.dt_bias[h * DK + c0 + u];
    }
    for (int64_t t = t0 + rg; t < t_end; t += RPI) {
        const int64_t row = t * a.H + h, e = row * DK + c0;
        float q[8], k[8], g[8];
        load8(static_cast<const Tin*>(a.q_raw), e, q);
        load8(static_cast<const Tin*>(a.k_raw), e, k);
        load8(static_cast<const Tin*>(a.g_logit), e, g);
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            sq += q[u] * q[u];
            sk += k[u] * k[u];
        }
        sq = group_sum<L>(sq);
        sk = group_sum<L>(sk);
        const float rq = 1.f / sqrtf(sq + a.l2_eps), rk = 1.f / sqrtf(sk + a.l2_eps);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            q[u] *= rq;
            k[u] *= rk;
            g[u] = a.gate_lb * sigmoid(eA[u] * (g[u] + bias[u]));
        }
        store8(reinterpret_cast<Tout*>(a.qf), e, q);
        store8(reinterpret_cast<Tout*>(a.kf), e, k);
        store8(reinterpret_cast<Tout*>(a.gf), e, g);
        if (part == 0)
            store_elem(reinterpret_cast<Tout*>(a.bf), row,
                       sigmoid(load_elem(static_cast<const Tin*>(a.beta_logit), row)));
    }
    // v and dO widened to float32 (for the vector-ALU backward): Dv/8 lanes per row
    if (!a.widen_x) return;
    const int LV = a.Dv / 8, RV = kPThreads / LV;
    const int pv = tid % LV, rv = tid / LV;
    if (rv < RV) {
        for (int64_t t = t0 + rv; t < t_end; t += RV) {
            const int64_t e = (t * a.H + h) * a.Dv + 8 * pv;
            float x[8];
            load8(static_cast<const Tin*>(a.v), e, x);
            store8(a.vf, e, x);
            load8(static_cast<const Tin*>(a.d_o), e, x);
            store8(a.dof, e, x);
        }
    }
}

template <typename Tin, int DK>
__global__ __launch_bounds__(kPThreads) void prologue_grad_kernel(PrologueBwdArgs a) {
    constexpr int L = DK / 8, RPI = kPThreads / L;
    __shared__ float red[2][RPI][DK + 1];
    const int tid = threadIdx.x, part = tid % L, rg = tid / L, c0 = 8 * part;
    const int h = blockIdx.y;
    const int64_t rows_total = (int64_t)a.B * a.T;
    const int64_t t0 = (int64_t)blockIdx.x * kTokBlock;
    const int64_t t_end = min(t0 + kTokBlock, rows_total);
    float eA[8], bias[8], acc_b[8], acc_A[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        eA[u] = __expf(a.A_log[c0 + u]);
        bias[u] = a.dt_bias[h * DK + c0 + u];
        acc_b[u] = acc_A[u] = 0.f;
    }
    for (int64_t t = t0 + rg; t < t_end; t += RPI) {
        const int64_t row = t * a.H + h, e = row * DK + c0;
        float q[8], k[8], g[8], dq[8], dk[8], dg[8];
        load8(static_cast<const Tin*>(a.q_raw), e, q);
        load8(static_cast<const Tin*>(a.k_raw), e, k);
        load8(static_cast<const Tin*>(a.g_logit), e, g);
        load8(a.dq, e, dq);
        load8(a.dk, e, dk);
        load8(a.dg, e, dg);
        float sq = 0.f, pq = 0.f, sk = 0.f, pk = 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            sq += q[u] * q[u];
            pq += q[u] * dq[u];
            sk += k[u] * k[u];
            pk += k[u] * dk[u];
        }
        sq = group_sum<L>(sq);
        pq = group_sum<L>(pq);
        sk = group_sum<L>(sk);
        pk = group_sum<L>(pk);
        const float nq = sqrtf(sq + a.l2_eps), nk = sqrtf(sk + a.l2_eps);
        const float cq = pq / (nq * nq * nq), ck = pk / (nk * nk * nk);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            dq[u] = dq[u] / nq - q[u] * cq;
            dk[u] = dk[u] / nk - k[u] * ck;
            const float z = eA[u] * (g[u] + bias[u]);
            const float sg = sigmoid(z);
            const float dz = dg[u] * a.gate_lb * sg * (1.f - sg);
            dg[u] = dz * eA[u];
            acc_b[u] += dz * eA[u];
            acc_A[u] += dz * z;
        }
        store8(a.dq, e, dq);
        store8(a.dk, e, dk);
        store8(a.dg, e, dg);
        if (part == 0) {
            const float sb = sigmoid(load_elem(static_cast<const Tin*>(a.beta_logit), row));
            a.dbeta[row] = a.dbeta[row] * sb * (1.f - sb);
        }
    }
    // per-channel sums over this workgroup's row groups, in a fixed order
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        red[0][rg][c0 + u] = acc_b[u];
        red[1][rg][c0 + u] = acc_A[u];
    }
    __syncthreads();
    if (tid < 2 * DK) {
        const int which = tid / DK, c = tid % DK;
        float acc = 0.f;
        for (int r = 0; r < RPI; ++r) acc += red[which][r][c];
        const int64_t p = ((int64_t)blockIdx.x * a.H + h) * DK + c;
        (which == 0 ? a.part_b : a.part_A)[p] = acc;
    }
}

// ddt_bias[h][c] = sum over token blocks (one thread per output), and
// dA_log[c] = sum over token blocks and heads (one workgroup per channel:
// strided partial sums, then a tree in LDS). Both in a fixed order.
__global__ void prologue_reduce_bias_kernel(PrologueBwdArgs a, int nblk, int DK) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= a.H * DK) return;
    const int h = i / DK, c = i % DK;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    int b = 0;
    for (; b + 4 <= nblk; b += 4)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] += a.part_b[((int64_t)(b + u) * a.H + h) * DK + c];
    for (; b < nblk; ++b) acc[0] += a.part_b[((int64_t)b * a.H + h) * DK + c];
    a.d_dt_bias[i] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

__global__ __launch_bounds__(256) void prologue_reduce_alog_kernel(PrologueBwdArgs a, int nblk, int DK) {
    __shared__ float red[256];
    const int c = blockIdx.x;
    const int64_t n = (int64_t)nblk * a.H;   // (token block, head) pairs
    float acc = 0.f;
    for (int64_t i = threadIdx.x; i < n; i += 256) acc += a.part_A[i * DK + c];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int m = 128; m >= 1; m >>= 1) {
        if ((int)threadIdx.x < m) red[threadIdx.x] += red[threadIdx.x + m];
        __syncthreads();
    }
    if (threadIdx.x == 0) a.d_A_log[c] = red[0];
}

// grad: the chain-rule pass; otherwise the apply pass, with outputs in float32
// or (same) in the input dtype
template <typename Tin>
hipError_t launch_apply(const PrologueBwdArgs& a, dim3 grid, hipStream_t s, bool grad, bool same = false) {
    const dim3 block(kPThreads);
    switch (a.Dk) {
        case 16:
            if (grad) prologue_grad_kernel<Tin, 16><<<grid, block, 0, s>>>(a);
            else if (same) prologue_apply_kernel<Tin, Tin, 16><<<grid, block, 0, s>>>(a);
            else prologue_apply_kernel<Tin, float, 16><<<grid, block, 0, s>>>(a);
            break;
        case 32:
            if (grad) prologue_grad_kernel<Tin, 32><<<grid, block, 0, s>>>(a);
            else if (same) prologue_apply_kernel<Tin, Tin, 32><<<grid, block, 0, s>>>(a);
            else prologue_apply_kernel<Tin, float, 32><<<grid, block, 0, s>>>(a);
            break;
        case 64:
            if (grad) prologue_grad_kernel<Tin, 64><<<grid, block, 0, s>>>(a);
            else if (same) prologue_apply_kernel<Tin, Tin, 64><<<grid, block, 0, s>>>(a);
            else prologue_apply_kernel<Tin, float, 64><<<grid, block, 0, s>>>(a);
            break;
        default:
            if (grad) prologue_grad_kernel<Tin, 128><<<grid, block, 0, s>>>(a);
            else if (same) prologue_apply_kernel<Tin, Tin, 128><<<grid, block, 0, s>>>(a);
            else prologue_apply_kernel<Tin, float, 128><<<grid, block, 0, s>>>(a);
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
    }
    // (with no tokens the reductions over zero token blocks write zeros)
    prologue_reduce_bias_kernel<<<dim3((unsigned)((p.H * p.Dk + 255) / 256)), dim3(256), 0, s>>>(p, (int)nblk, p.Dk);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    prologue_reduce_alog_kernel<<<dim3((unsigned)p.Dk), dim3(256), 0, s>>>(p, (int)nblk, p.Dk);
    return hipGetLastError();
}

hipError_t launch_prologue(const PrologueBwdArgs& p, hipStream_t s) {
    const int64_t nblk = prologue_bwd_token_blocks(p.B, p.T);
    if (nblk == 0) return hipSuccess;
    const dim3 grid((unsigned)nblk, (unsigned)p.H);
    return p.bf16 ? launch_apply<__bf16>(p, grid, s, false, true) : launch_apply<float>(p, grid, s, false, true);
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
