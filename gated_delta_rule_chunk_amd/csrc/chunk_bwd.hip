// Chunkwise KDA backward, all arithmetic in float32: a vector-ALU path for
// every supported head size (this part of the file) and a matrix-core path
// for d_k = 128 (namespace mf below).
//
// Loss: L = sum_t <dO_t, o_t> + <dS_final, S_final>. The forward's chunk form
// (16-row chunks, Gamma = in-chunk cumulative log-decay per channel, entry
// state S):
//   KK[r][s] = sum_c k_rc k_sc e^(Gamma_rc - Gamma_sc)         (s < r)
//   P[r][s]  = sum_c q_rc k_sc e^(Gamma_rc - Gamma_sc)         (s <= r)
//   T = (I + Diag(beta) KK)^-1,  W = V - Kg S,  U = T Diag(beta) W
//   O = scale (Qh S + P U),  S_next = Diag(e^Gamma_C) S + Kh^T U
// with Kg = e^Gamma * K, Qh = e^Gamma * Q, Kh = e^(Gamma_C - Gamma) * K.
// Differentiating it, with dS the gradient at the chunk's end:
//   dU = scale P^T dO + Kh dS,   dY = T^T dU,   dW = Diag(beta) dY = dV
//   dP = scale dO U^T (lower),   dM = -dY U^T (strict lower),  dKK = Diag(beta) dM
//   dbeta_r = dY_r . W_r + sum_s dM[r][s] KK[r][s]
//   dS_prev = Diag(e^Gamma_C) dS + scale Qh^T dO - Kg^T dW
// then through the exponentials to dq, dk and dGamma channel by channel,
// every pair term differentiated with its own e^(Gamma_r - Gamma_s) (only
// exponentials of differences, as in the forward); dg is the reverse
// cumulative sum of dGamma over the chunk, Gamma_C's gradient entering at
// its last row.
//
// Vector-ALU path, two kernels: chunk_states_kernel re-runs the forward and
// writes each chunk's entry state to a caller-provided workspace;
// chunk_bwd_kernel walks every sequence backward from its last chunk. Both own one (sequence, head,
// value slice of up to 64 columns). The slices' partial sums of dq, dk, dg
// and dbeta meet in float32 atomic adds onto zeroed outputs; with two slices
// (d_v = 128) the sum does not depend on their order.
#include "device_common.hpp"
#include "launchers.hpp"

namespace kda {
namespace {

constexpr int kBC = 16;  // chunk rows
constexpr int kBwdThreads = 512;
constexpr int kWaves = kBwdThreads / 64;
constexpr int kPairs = kBC * (kBC + 1) / 2;

struct SeqInfo {
    int64_t bos, len, b, slot0;
};

__device__ __forceinline__ SeqInfo seq_info(const BwdArgs& a, int n) {
    SeqInfo s;
    if (a.cu) {
        s.bos = a.cu[n];
        s.len = (int64_t)a.cu[n + 1] - s.bos;
        s.b = 0;
        s.slot0 = s.bos / kBC + n;
    } else {
        s.bos = 0;
        s.len = a.T;
        s.b = n;
        s.slot0 = (int64_t)n * ((a.T + kBC - 1) / kBC);
    }
    return s;
}

// Pair index p = r(r+1)/2 + s (s <= r) -> (r, s).
__device__ __forceinline__ void pair_rs(int p, int& r, int& s) {
    int rr = (int)((__builtin_sqrtf(8.f * p + 1.f) - 1.f) * 0.5f);
    if ((rr + 1) * (rr + 2) / 2 <= p) ++rr;
    if (rr * (rr + 1) / 2 > p) --rr;
    r = rr;
    s = p - rr * (rr + 1) / 2;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

__device__ __forceinline__ void add_out(float* p, float v, bool atomic) {
    if (atomic)
        unsafeAtomicAdd(p, v);
    else
        *p = v;
}

// One chunk's K (and Q when sQ is given), the log2-scaled gate and beta;
// rows past the sequence's end are zero tokens.
template <int DK, typename Tin>
__device__ __forceinline__ void load_chunk(const BwdArgs& a, const SeqInfo& sq, int h, int64_t t0,
                                           int rows, float (*sQ)[DK], float (*sK)[DK],
                                           float (*sG)[DK], float* sBeta) {
    const Tin* q = static_cast<const Tin*>(a.q);
    const Tin* k = static_cast<const Tin*>(a.k);
    const Tin* g = static_cast<const Tin*>(a.g);
    const Tin* beta = static_cast<const Tin*>(a.beta);
    for (int idx = threadIdx.x; idx < kBC * DK; idx += kBwdThreads) {
        const int r = idx / DK, c = idx % DK;
        const bool in = r < rows;
        const int64_t e = ((sq.b * a.T + t0 + r) * a.H + h) * DK + c;
        if (sQ) sQ[r][c] = in ? load_elem(q, e) : 0.f;
        sK[r][c] = in ? load_elem(k, e) : 0.f;
        sG[r][c] = in ? load_elem(g, e) * kLog2e : 0.f;
    }
    if (threadIdx.x < kBC) {
        const int r = threadIdx.x;
        sBeta[r] = r < rows ? load_elem(beta, (sq.b * a.T + t0 + r) * a.H + h) : 0.f;
    }
}

// Rows of [C][BV] from a [.., H, Dv] tensor, columns c0 .. c0+BV.
template <int BV, typename Tin>
__device__ __forceinline__ void load_rows_v(const Tin* x, const BwdArgs& a, const SeqInfo& sq, int h,
                                            int64_t t0, int rows, int c0, float (*dst)[BV]) {
    for (int idx = threadIdx.x; idx < kBC * BV; idx += kBwdThreads) {
        const int r = idx / BV, j = idx % BV;
        dst[r][j] = r < rows ? load_elem(x, ((sq.b * a.T + t0 + r) * a.H + h) * a.Dv + c0 + j) : 0.f;
    }
}

// In-chunk cumulative sum of the (log2-scaled) gate per channel, and
// e^Gamma_C; then Kg, Kh (and Qh) for every (row, channel).
template <int DK>
__device__ __forceinline__ void gamma_and_scaled(float (*sG)[DK], float* sEC, const float (*sQ)[DK],
                                                 const float (*sK)[DK], float (*sQh)[DK],
                                                 float (*sKg)[DK], float (*sKh)[DK]) {
    if (threadIdx.x < DK) {
        const int c = threadIdx.x;
        float run = 0.f;
#pragma unroll
        for (int r = 0; r < kBC; ++r) {
            run += sG[r][c];
            sG[r][c] = run;
        }
        sEC[c] = __builtin_amdgcn_exp2f(run);
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < kBC * DK; idx += kBwdThreads) {
        const int r = idx / DK, c = idx % DK;
        const float gr = sG[r][c];
        const float e = __builtin_amdgcn_exp2f(gr);
        const float k = sK[r][c];
        if (sQh) sQh[r][c] = e * sQ[r][c];
        sKg[r][c] = e * k;
        sKh[r][c] = __builtin_amdgcn_exp2f(sG[kBC - 1][c] - gr) * k;
    }
}

// KK (strict lower) and, when sP is given, P (lower with diagonal): one wave
// per (r, s) pair, lanes across channels.
template <int DK>
__device__ __forceinline__ void pair_sums(const float (*sG)[DK], const float (*sK)[DK],
                                          const float (*sQ)[DK], float (*sKK)[kBC + 1],
                                          float (*sP)[kBC + 1]) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int p = w; p < kPairs; p += kWaves) {
        int r, s;
        pair_rs(p, r, s);
        if (!sP && s == r) continue;
        float ak = 0.f, ap = 0.f;
        for (int c = lane; c < DK; c += 64) {
            const float e = __builtin_amdgcn_exp2f(sG[r][c] - sG[s][c]);
            const float ks = sK[s][c] * e;
            ak += sK[r][c] * ks;
            if (sP) ap += sQ[r][c] * ks;
        }
        ak = wave_sum(ak);
        if (sP) ap = wave_sum(ap);
        if (lane == 0) {
            sKK[r][s] = s < r ? ak : 0.f;
            if (sP) sP[r][s] = ap;
        }
    }
}

// T = (I + Diag(beta) KK)^-1 (unit lower triangular), one thread per column.
__device__ __forceinline__ void invert_unit_lower(const float (*sKK)[kBC + 1], const float* sBeta,
                                                  float (*sT)[kBC + 1]) {
    if (threadIdx.x < kBC) {
        const int i = threadIdx.x;
        for (int r = 0; r < kBC; ++r) {
            float t;
            if (r < i) {
                t = 0.f;
            } else if (r == i) {
                t = 1.f;
            } else {
                float acc = 0.f;
                for (int s = i; s < r; ++s) acc += sKK[r][s] * sT[s][i];
                t = -sBeta[r] * acc;
            }
            sT[r][i] = t;
        }
    }
}

template <int DK, int BV, typename Tin>
__global__ __launch_bounds__(kBwdThreads) void chunk_states_kernel(BwdArgs a) {
    __shared__ float sS[DK][BV + 1];
    __shared__ float sK[kBC][DK];
    __shared__ float sG[kBC][DK];
    __shared__ float sKg[kBC][DK];
    __shared__ float sKh[kBC][DK];
    __shared__ float sW[kBC][BV];
    __shared__ float sU[kBC][BV];
    __shared__ float sKK[kBC][kBC + 1];
    __shared__ float sT[kBC][kBC + 1];
    __shared__ float sBeta[kBC];
    __shared__ float sEC[DK];

    const int tid = threadIdx.x;
    const int nvt = a.Dv / BV;
    const int vt = blockIdx.x % nvt, unit = blockIdx.x / nvt;
    const int n = unit / a.H, h = unit % a.H;
    const int Dv = a.Dv, c0 = vt * BV;
    const SeqInfo sq = seq_info(a, n);
    const int64_t sbase = ((int64_t)n * a.H + h) * DK * (int64_t)Dv;
    const int64_t slot_stride = (int64_t)a.H * DK * Dv;

    for (int idx = tid; idx < DK * BV; idx += kBwdThreads) {
        const int c = idx / BV, j = idx % BV;
        sS[c][j] = a.s0 ? a.s0[sbase + (int64_t)c * Dv + c0 + j] : 0.f;
    }
    __syncthreads();
    const int64_t nch = (sq.len + kBC - 1) / kBC;
    for (int64_t ch = 0; ch < nch; ++ch) {
        const int64_t t0 = sq.bos + ch * kBC;
        const int rows = (int)min<int64_t>(kBC, sq.len - ch * kBC);
        float* ws = a.ws + (sq.slot0 + ch) * slot_stride + (int64_t)h * DK * Dv;
        for (int idx = tid; idx < DK * BV; idx += kBwdThreads) {
            const int c = idx / BV, j = idx % BV;
            ws[(int64_t)c * Dv + c0 + j] = sS[c][j];
        }
        load_chunk<DK, Tin>(a, sq, h, t0, rows, nullptr, sK, sG, sBeta);
        load_rows_v<BV>(static_cast<const Tin*>(a.v), a, sq, h, t0, rows, c0, sW);
        __syncthreads();
        gamma_and_scaled<DK>(sG, sEC, nullptr, sK, nullptr, sKg, sKh);
        pair_sums<DK>(sG, sK, nullptr, sKK, nullptr);
        __syncthreads();
        invert_unit_lower(sKK, sBeta, sT);
        // W = V - Kg S (in place)
        for (int idx = tid; idx < kBC * BV; idx += kBwdThreads) {
            const int r = idx / BV, j = idx % BV;
            float acc = 0.f;
#pragma unroll 8
            for (int c = 0; c < DK; ++c) acc += sKg[r][c] * sS[c][j];
            sW[r][j] -= acc;
        }
        __syncthreads();
        // U = T Diag(beta) W
        for (int idx = tid; idx < kBC * BV; idx += kBwdThreads) {
            const int r = idx / BV, j = idx % BV;
            float acc = 0.f;
            for (int s = 0; s <= r; ++s) acc += sT[r][s] * sBeta[s] * sW[s][j];
            sU[r][j] = acc;
        }
        __syncthreads();
        // S <- Diag(e^Gamma_C) S + Kh^T U
        for (int idx = tid; idx < DK * BV; idx += kBwdThreads) {
            const int c = idx / BV, j = idx % BV;
            float acc = sEC[c] * sS[c][j];
#pragma unroll
            for (int r = 0; r < kBC; ++r) acc += sKh[r][c] * sU[r][j];
            sS[c][j] = acc;
        }
        __syncthreads();
    }
}

template <int DK, int BV, typename Tin>
__global__ __launch_bounds__(kBwdThreads) void chunk_bwd_kernel(BwdArgs a) {
    constexpr int kGroups = kBwdThreads / DK;  // threads sharing one channel
    static_assert(kBwdThreads % DK == 0, "each thread keeps one channel");
    __shared__ float sS[DK][BV + 1];
    __shared__ float sdS[DK][BV + 1];
    __shared__ float sQ[kBC][DK];
    __shared__ float sK[kBC][DK];
    __shared__ float sG[kBC][DK];
    __shared__ float sQh[kBC][DK];
    __shared__ float sKg[kBC][DK];
    __shared__ float sKh[kBC][DK];
    __shared__ float sdG[kBC][DK];
    __shared__ float sW[kBC][BV];
    __shared__ float sU[kBC][BV];
    __shared__ float sdO[kBC][BV];
    __shared__ float sdUW[kBC][BV];  // dU, then dW
    __shared__ float sdY[kBC][BV];
    __shared__ float sKK[kBC][kBC + 1];
    __shared__ float sP[kBC][kBC + 1];
    __shared__ float sT[kBC][kBC + 1];
    __shared__ float sdP[kBC][kBC + 1];
    __shared__ float sdM[kBC][kBC + 1];
    __shared__ float sBeta[kBC];
    __shared__ float sEC[DK];
    __shared__ float sGCp[kGroups][DK];
    __shared__ float sGC0[DK];

    const Tin* v = static_cast<const Tin*>(a.v);
    const Tin* d_o = static_cast<const Tin*>(a.d_o);
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int nvt = a.Dv / BV;
    const bool atomic = nvt > 1;
    const int vt = blockIdx.x % nvt, unit = blockIdx.x / nvt;
    const int n = unit / a.H, h = unit % a.H;
    const int H = a.H, Dv = a.Dv, c0 = vt * BV;
    const float scale = a.scale;
    const SeqInfo sq = seq_info(a, n);
    const int64_t sbase = ((int64_t)n * H + h) * DK * (int64_t)Dv;
    const int64_t slot_stride = (int64_t)H * DK * Dv;

    for (int idx = tid; idx < DK * BV; idx += kBwdThreads) {
        const int c = idx / BV, j = idx % BV;
        sdS[c][j] = a.d_final ? a.d_final[sbase + (int64_t)c * Dv + c0 + j] : 0.f;
    }
    const int64_t nch = (sq.len + kBC - 1) / kBC;
    for (int64_t ch = nch - 1; ch >= 0; --ch) {
        const int64_t t0 = sq.bos + ch * kBC;
        const int rows = (int)min<int64_t>(kBC, sq.len - ch * kBC);
        const float* ws = a.ws + (sq.slot0 + ch) * slot_stride + (int64_t)h * DK * Dv;
        for (int idx = tid; idx < DK * BV; idx += kBwdThreads) {
            const int c = idx / BV, j = idx % BV;
            sS[c][j] = ws[(int64_t)c * Dv + c0 + j];
        }
        load_chunk<DK, Tin>(a, sq, h, t0, rows, sQ, sK, sG, sBeta);
        load_rows_v<BV>(v, a, sq, h, t0, rows, c0, sW);
        load_rows_v<BV>(d_o, a, sq, h, t0, rows, c0, sdO);
        __syncthreads();
        gamma_and_scaled<DK>(sG, sEC, sQ, sK, sQh, sKg, sKh);
        pair_sums<DK>(sG, sK, sQ, sKK, sP);
        __syncthreads();
        invert_unit_lower(sKK, sBeta, sT);
        // W = V - Kg S (in place);  dU = scale P^T dO + Kh dS
        for (int idx = tid; idx < kBC * BV; idx += kBwdThreads) {
            const int r = idx / BV, j = idx % BV;
            float aw = 0.f, au = 0.f;
#pragma unroll 8
            for (int c = 0; c < DK; ++c) {
                aw += sKg[r][c] * sS[c][j];
                au += sKh[r][c] * sdS[c][j];
            }
            float ap = 0.f;
            for (int s = r; s < kBC; ++s) ap += sP[s][r] * sdO[s][j];
            sW[r][j] -= aw;
            sdUW[r][j] = au + scale * ap;
        }
        __syncthreads();
        // U = T Diag(beta) W;  dY = T^T dU
        for (int idx = tid; idx < kBC * BV; idx += kBwdThreads) {
            const int r = idx / BV, j = idx % BV;
            float au = 0.f, ay = 0.f;
            for (int s = 0; s <= r; ++s) au += sT[r][s] * sBeta[s] * sW[s][j];
            for (int s = r; s < kBC; ++s) ay += sT[s][r] * sdUW[s][j];
            sU[r][j] = au;
            sdY[r][j] = ay;
        }
        __syncthreads();
        // dP = scale dO U^T (s <= r), dM = -dY U^T (s < r): one wave per pair
        for (int p = w; p < kPairs; p += kWaves) {
            int r, s;
            pair_rs(p, r, s);
            float ap = 0.f, am = 0.f;
            for (int j = lane; j < BV; j += 64) {
                const float us = sU[s][j];
                ap += sdO[r][j] * us;
                am += sdY[r][j] * us;
            }
            ap = wave_sum(ap);
            am = wave_sum(am);
            if (lane == 0) {
                sdP[r][s] = scale * ap;
                sdM[r][s] = s < r ? -am : 0.f;
            }
        }
        // dW = Diag(beta) dY = dV
        for (int idx = tid; idx < kBC * BV; idx += kBwdThreads) {
            const int r = idx / BV, j = idx % BV;
            const float dw = sBeta[r] * sdY[r][j];
            sdUW[r][j] = dw;
            if (r < rows) a.dv[((sq.b * a.T + t0 + r) * H + h) * (int64_t)Dv + c0 + j] = dw;
        }
        __syncthreads();
        // dbeta
        if (tid < kBC && tid < rows) {
            const int r = tid;
            float acc = 0.f;
            for (int j = 0; j < BV; ++j) acc += sdY[r][j] * sW[r][j];
            for (int s = 0; s < r; ++s) acc += sdM[r][s] * sKK[r][s];
            add_out(a.dbeta + (sq.b * a.T + t0 + r) * H + h, acc, atomic);
        }
        // dq, dk and dGamma per (row, channel)
        {
            const int c = tid % DK;
            float gc_part = 0.f;
            for (int idx = tid; idx < kBC * DK; idx += kBwdThreads) {
                const int r = idx / DK;
                const float gr = sG[r][c], qr = sQ[r][c], kr = sK[r][c];
                // pairs with this row as the later one (r, s <= r)
                float accq = 0.f, acckr = 0.f;
                for (int s = 0; s <= r; ++s) {
                    const float ks = sK[s][c] * __builtin_amdgcn_exp2f(gr - sG[s][c]);
                    accq += sdP[r][s] * ks;
                    acckr += sBeta[r] * sdM[r][s] * ks;
                }
                // pairs with this row as the earlier one (r2 >= r, r)
                float accks = 0.f;
                for (int r2 = r; r2 < kBC; ++r2) {
                    const float e = __builtin_amdgcn_exp2f(sG[r2][c] - gr);
                    accks += (sdP[r2][r] * sQ[r2][c] + sBeta[r2] * sdM[r2][r] * sK[r2][c]) * e;
                }
                // dense terms
                float ao = 0.f, aw = 0.f, ad = 0.f;
#pragma unroll 8
                for (int j = 0; j < BV; ++j) {
                    const float sv = sS[c][j];
                    ao += sdO[r][j] * sv;
                    aw += sdUW[r][j] * sv;
                    ad += sU[r][j] * sdS[c][j];
                }
                const float qh = sQh[r][c], kg = sKg[r][c], kh = sKh[r][c];
                const float eg = __builtin_amdgcn_exp2f(gr);
                const float eh = __builtin_amdgcn_exp2f(sG[kBC - 1][c] - gr);
                const float dqv = accq + eg * scale * ao;
                const float dkv = acckr + accks - eg * aw + eh * ad;
                const float dgv = qr * accq + kr * acckr - kr * accks + qh * scale * ao - kg * aw - kh * ad;
                gc_part += kh * ad;
                sdG[r][c] = dgv;
                if (r < rows) {
                    const int64_t e = ((sq.b * a.T + t0 + r) * H + h) * DK + c;
                    add_out(a.dq + e, dqv, atomic);
                    add_out(a.dk + e, dkv, atomic);
                }
            }
            sGCp[tid / DK][c] = gc_part;
            if (tid < DK) {
                float acc = 0.f;
                for (int j = 0; j < BV; ++j) acc += sdS[c][j] * sS[c][j];
                sGC0[c] = sEC[c] * acc;
            }
        }
        __syncthreads();
        // dg: reverse cumulative sum of dGamma, Gamma_C's gradient at the last row
        if (tid < DK) {
            const int c = tid;
            float run = sGC0[c];
            for (int p = 0; p < kGroups; ++p) run += sGCp[p][c];
            for (int r = kBC - 1; r >= 0; --r) {
                run += sdG[r][c];
                if (r < rows) add_out(a.dg + ((sq.b * a.T + t0 + r) * H + h) * DK + c, run, atomic);
            }
        }
        // dS <- Diag(e^Gamma_C) dS + scale Qh^T dO - Kg^T dW
        for (int idx = tid; idx < DK * BV; idx += kBwdThreads) {
            const int c = idx / BV, j = idx % BV;
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < kBC; ++r) acc += scale * sQh[r][c] * sdO[r][j] - sKg[r][c] * sdUW[r][j];
            sdS[c][j] = sEC[c] * sdS[c][j] + acc;
        }
        __syncthreads();
    }
    if (a.d_s0) {
        for (int idx = tid; idx < DK * BV; idx += kBwdThreads) {
            const int c = idx / BV, j = idx % BV;
            a.d_s0[sbase + (int64_t)c * Dv + c0 + j] = sdS[c][j];
        }
    }
}

__global__ void zero_fill_kernel(float* p, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0.f;
}

hipError_t zero_fill(float* p, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
    zero_fill_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p, n);
    return hipGetLastError();
}

template <int DK, int BV, typename Tin>
hipError_t launch_typed(const BwdArgs& a, hipStream_t s) {
    const int64_t grid = (int64_t)a.N * a.H * (a.Dv / BV);
    if (grid == 0) return hipSuccess;
    chunk_states_kernel<DK, BV, Tin><<<dim3((unsigned)grid), dim3(kBwdThreads), 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    chunk_bwd_kernel<DK, BV, Tin><<<dim3((unsigned)grid), dim3(kBwdThreads), 0, s>>>(a);
    return hipGetLastError();
}

// Value columns per workgroup: d_v = 64 in two 32-column slices (twice the
// workgroups of one 64-column slice; with two slices each atomically summed
// gradient gets exactly two addends, so the sums do not depend on their
// order), 64-column slices for d_v = 128, all of d_v below 64.
constexpr int vbwd_bv(int Dv) { return Dv == 64 ? 32 : (Dv > 64 ? 64 : Dv); }

template <int DK, typename Tin>
hipError_t launch_dk(const BwdArgs& a, hipStream_t s) {
    switch (a.Dv) {
        case 16: return launch_typed<DK, 16, Tin>(a, s);
        case 32:
        case 64: return launch_typed<DK, 32, Tin>(a, s);
        default: return launch_typed<DK, 64, Tin>(a, s);  // 128
    }
}

template <typename Tin>
hipError_t launch_dtype(const BwdArgs& a, hipStream_t s) {
    switch (a.Dk) {
        case 16: return launch_dk<16, Tin>(a, s);
        case 32: return launch_dk<32, Tin>(a, s);
        case 64: return launch_dk<64, Tin>(a, s);
        default: return launch_dk<128, Tin>(a, s);
    }
}


// ---------------------------------------------------------------------------
// Matrix-core variant for d_k = 128 and 64-column value slices.
//
// Same chunk algebra as above; every dense product with the state or its
// gradient (W = V - Kg S, Kh dS, dO S^T, dW S^T, U dS^T, the state and
// state-gradient updates) and the small 16x16 products (T W, T^T dU, dO U^T,
// dY U^T, dY W^T) run on v_mfma_f32_16x16x4f32, which takes float32
// operands, so the arithmetic stays float32. One workgroup of 8 waves owns
// (sequence, head, slice): it first re-runs the forward over the sequence,
// writing each chunk's entry state to the workspace, then walks the chunks
// backward. Wave w keeps rows 16w..16w+15 of the state (forward sweep) and of
// the state gradient (backward sweep) in registers, in the MFMA result layout
// (lane l: rows 16w + 4(l/16) + i, column 16t + l%16 of tile t).
//
// f32 16x16x4 operand layouts (lane l, l16 = l%16, lg = l/16): A[m][k] with
// m = l16, k = lg; B[k][n] with k = lg, n = l16; D[m][n] with m = 4lg + i
// (register i), n = l16.
namespace mf {

constexpr int C = 16, DK = 128, BV = 64, NT = 512;
constexpr int SP = BV + 4;   // row stride of the [DK][SP] state tiles
constexpr int KP = DK + 2;   // row stride of [C][KP] per-channel rows (= 2 mod 32: operand reads by row hit distinct banks)
constexpr int VP = BV + 2;   // row stride of [C][VP] per-column rows (likewise)
constexpr int CP = C + 1;
constexpr int kRef = 7;      // reference row of the factored pair exponentials
constexpr int kMats = 3 * C * C;   // T, P, KK of one chunk

struct Smem {
    float S[DK][SP];
    float dS[DK][SP];
    float G[C][KP];
    float Qh[C][KP], Kg[C][KP], Kh[C][KP], Qp[C][KP], Kp[C][KP], Km[C][KP];
    float W[C][VP], U[C][VP], dO[C][VP], dUW[C][VP], dY[C][VP];
    float KK[C][CP], P[C][CP], T[C][CP], dP[C][CP], dKK[C][CP];
    float beta[C], EC[DK];
    float dbp[C], xd[C];   // the two parts of dbeta
};

__device__ __forceinline__ f32x4 mfma(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Sum over the 16 lanes of each row of the wave (DPP row shifts); lane 15 of
// each row ends with the row's total.
__device__ __forceinline__ float row16_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, true));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, true));
    return v;
}

// Four consecutive input elements, raw (float4 or four bf16 in a uint2).
template <typename T> struct Raw4;
template <> struct Raw4<float> {
    float4 v;
    __device__ __forceinline__ void load(const float* p, int64_t i) { v = *reinterpret_cast<const float4*>(p + i); }
    __device__ __forceinline__ float get(int u) const { return u == 0 ? v.x : u == 1 ? v.y : u == 2 ? v.z : v.w; }
};
// One element, raw: converted when it is used, not when it is loaded (a
// conversion right after the load would wait for the data there and hold up
// every load issued after it).
template <typename T> struct Raw1;
template <> struct Raw1<float> {
    float v;
    __device__ __forceinline__ void load(const float* p, int64_t i) { v = p[i]; }
    __device__ __forceinline__ float get() const { return v; }
};
template <> struct Raw1<__bf16> {
    uint16_t v;
    __device__ __forceinline__ void load(const __bf16* p, int64_t i) { v = reinterpret_cast<const uint16_t*>(p)[i]; }
    __device__ __forceinline__ float get() const { return __uint_as_float((uint32_t)v << 16); }
};
template <> struct Raw4<__bf16> {
    uint2 v;
    __device__ __forceinline__ void load(const __bf16* p, int64_t i) {
        v = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(p) + i);
    }
    __device__ __forceinline__ float get(int u) const {
        const uint32_t w = u < 2 ? v.x : v.y;
        return __uint_as_float((u & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};

// One chunk's global inputs held in registers between issue and commit, so
// that every load of a chunk is in flight at once. They are issued in the
// order they are committed: q, k, g and beta (which the scaling phase needs)
// first, then v or dO, T/P/KK and the entry state, which the reverse sweep
// commits only after the scaling phase, while they are still arriving. Rows
// past the sequence's end load row 0 (always in range) and are zeroed at
// commit.
template <typename Tin, typename Tx>
struct Fetch {
    Raw4<Tin> q, k, g;
    Raw4<Tx> x;             // x: v for threads < 256, dO for the others
    Raw1<Tin> beta;
    float4 s[4];            // entry state slice (reverse sweep)
    float m[3];             // T, P, KK entries (threads < 256)
    bool in_qk, in_x, in_b;
};

template <typename Tin, typename Tx>
__device__ __forceinline__ void fetch_chunk(Fetch<Tin, Tx>& f, const BwdArgs& a, const SeqInfo& sq, int h, int64_t t0,
                                            int rows, int c0, bool reverse, const float* ws, const float* mats) {
    const int tid = threadIdx.x;
    {
        const int r = tid >> 5, c = (tid & 31) * 4;   // 16 rows x 32 quads
        f.in_qk = r < rows;
        const int64_t e = ((sq.b * a.T + t0 + (f.in_qk ? r : 0)) * a.H + h) * DK + c;
        f.k.load(static_cast<const Tin*>(a.k), e);
        f.g.load(static_cast<const Tin*>(a.g), e);
        if (reverse) f.q.load(static_cast<const Tin*>(a.q), e);
    }
    {
        const int r = tid & (C - 1);
        f.in_b = r < rows;
        f.beta.load(static_cast<const Tin*>(a.beta), (sq.b * a.T + t0 + (f.in_b ? r : 0)) * a.H + h);
    }
    {
        const int t2 = tid & 255;
        const int r = t2 >> 4, j = (t2 & 15) * 4;    // 16 rows x 16 quads
        f.in_x = r < rows;
        const int64_t e = ((sq.b * a.T + t0 + (f.in_x ? r : 0)) * a.H + h) * (int64_t)a.Dv + c0 + j;
        if (tid < 256)
            f.x.load(static_cast<const Tx*>(a.v), e);
        else if (reverse)
            f.x.load(static_cast<const Tx*>(a.d_o), e);
    }
    if (tid < C * C) {
        f.m[0] = mats[tid];
        if (reverse) {
            f.m[1] = mats[C * C + tid];
            f.m[2] = mats[2 * C * C + tid];
        }
    }
    if (reverse) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int q4 = tid + NT * u;             // 128 rows x 16 quads
            f.s[u] = *reinterpret_cast<const float4*>(ws + (int64_t)(q4 >> 4) * a.Dv + (q4 & 15) * 4);
        }
    }
}

// q, k, g and beta (what the scaling phase reads)
template <typename Tin, typename Tx>
__device__ __forceinline__ void commit_qkg(Smem& sm, const Fetch<Tin, Tx>& f, bool reverse) {
    const int tid = threadIdx.x;
    {
        const int r = tid >> 5, c = (tid & 31) * 4;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            sm.Kg[r][c + u] = f.in_qk ? f.k.get(u) : 0.f;
            sm.G[r][c + u] = f.in_qk ? f.g.get(u) * kLog2e : 0.f;
            if (reverse) sm.Qh[r][c + u] = f.in_qk ? f.q.get(u) : 0.f;
        }
    }
    if (tid < C) sm.beta[tid] = f.in_b ? f.beta.get() : 0.f;
}

// v or dO, T/P/KK and (reverse sweep) the entry state
template <typename Tin, typename Tx>
__device__ __forceinline__ void commit_rest(Smem& sm, const Fetch<Tin, Tx>& f, bool reverse) {
    const int tid = threadIdx.x;
    {
        const int t2 = tid & 255;
        const int r = t2 >> 4, j = (t2 & 15) * 4;
        if (tid < 256) {
#pragma unroll
            for (int u = 0; u < 4; ++u) sm.W[r][j + u] = f.in_x ? f.x.get(u) : 0.f;
        } else if (reverse) {
#pragma unroll
            for (int u = 0; u < 4; ++u) sm.dO[r][j + u] = f.in_x ? f.x.get(u) : 0.f;
        }
    }
    if (tid < C * C) {
        const int r = tid / C, s = tid % C;
        sm.T[r][s] = f.m[0];
        if (reverse) {
            sm.P[r][s] = f.m[1];
            sm.KK[r][s] = f.m[2];
        }
    }
    if (reverse) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int q4 = tid + NT * u;
            const int c = q4 >> 4, j = (q4 & 15) * 4;
            sm.S[c][j] = f.s[u].x; sm.S[c][j + 1] = f.s[u].y; sm.S[c][j + 2] = f.s[u].z; sm.S[c][j + 3] = f.s[u].w;
        }
    }
}

// Gamma (in-chunk cumulative log2 decay) and e^Gamma_C; then, per (row,
// channel), the scaled rows the products use:
//   Kg = e^Gamma k, Kh = e^(Gamma_C - Gamma) k, and in the reverse sweep
//   Qh = e^Gamma q, Qp = e^(Gamma - Gamma_ref) q, Kp = e^(Gamma - Gamma_ref) k,
//   Km = e^(Gamma_ref - Gamma) k
// with Gamma_ref the row kRef, so that e^(Gamma_r - Gamma_s) =
// e^(Gamma_r - Gamma_ref) e^(Gamma_ref - Gamma_s) turns the pair sums and
// their gradients into matrix products. With g >= -5 every exponent stays
// within 2^58.
__device__ __forceinline__ void chunk_scale(Smem& sm, bool reverse) {
    const int tid = threadIdx.x;
    if (tid < DK) {
        float run = 0.f;
#pragma unroll
        for (int r = 0; r < C; ++r) {
            run += sm.G[r][tid];
            sm.G[r][tid] = run;
        }
        sm.EC[tid] = __builtin_amdgcn_exp2f(run);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int idx = tid + NT * u;
        const int r = idx / DK, c = idx % DK;
        const float gr = sm.G[r][c];
        const float k = sm.Kg[r][c];
        const float eg = __builtin_amdgcn_exp2f(gr);
        sm.Kg[r][c] = eg * k;
        sm.Kh[r][c] = __builtin_amdgcn_exp2f(sm.G[C - 1][c] - gr) * k;
        if (reverse) {
            const float gref = sm.G[kRef][c];
            const float q = sm.Qh[r][c];
            const float ep = __builtin_amdgcn_exp2f(gr - gref);
            sm.Qh[r][c] = eg * q;
            sm.Qp[r][c] = ep * q;
            sm.Kp[r][c] = ep * k;
            sm.Km[r][c] = __builtin_amdgcn_exp2f(gref - gr) * k;
        }
    }
}

// W = V - Kg S for columns 16t..16t+15 (sm.W holds V on entry).
__device__ __forceinline__ void w_tile(Smem& sm, int t, int l16, int lg) {
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll 8
    for (int ks = 0; ks < DK / 4; ks += 2) {
        a0 = mfma(sm.Kg[l16][4 * ks + lg], sm.S[4 * ks + lg][16 * t + l16], a0);
        a1 = mfma(sm.Kg[l16][4 * ks + 4 + lg], sm.S[4 * ks + 4 + lg][16 * t + l16], a1);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.W[4 * lg + i][16 * t + l16] -= a0[i] + a1[i];
}

// U = T Diag(beta) W for columns 16t..16t+15.
__device__ __forceinline__ void u_tile(Smem& sm, int t, int l16, int lg) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C / 4; ++ks) {
        const int s = 4 * ks + lg;
        acc = mfma(sm.T[l16][s], sm.beta[s] * sm.W[s][16 * t + l16], acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.U[4 * lg + i][16 * t + l16] = acc[i];
}

// Per (chunk slot, head): T = (I + Diag(beta) KK)^-1, P and KK, which depend
// on q, k, g and beta only. Every chunk is independent, so this runs over all
// of them at once ahead of the sequential kernel.
struct MatsSmem {
    float G[C][KP], Qp[C][KP], Kp[C][KP], Km[C][KP];
    float KK[C][CP], beta[C];
};

template <typename Tin>
__global__ __launch_bounds__(256) void chunk_mats_kernel(BwdArgs a) {
    __shared__ MatsSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, lg = lane >> 4;
    const int64_t slot = blockIdx.x;
    const int h = blockIdx.y;
    int n;
    int64_t ch;
    if (a.cu) {   // largest n with cu[n]/16 + n <= slot
        int lo = 0, hi = a.N - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if ((int64_t)a.cu[mid] / C + mid <= slot) lo = mid; else hi = mid - 1;
        }
        n = lo;
        ch = slot - ((int64_t)a.cu[n] / C + n);
    } else {
        const int64_t per = (a.T + C - 1) / C;
        n = (int)(slot / per);
        ch = slot % per;
    }
    const SeqInfo sq = seq_info(a, n);
    if (ch * C >= sq.len) return;   // a slot no sequence uses (uniform per block)
    const int64_t t0 = sq.bos + ch * C;
    const int rows = (int)min<int64_t>(C, sq.len - ch * C);
    if (a.zero_grads) {
        // this chunk's rows of the atomically summed gradients: every token
        // row of every head lies in exactly one (slot, head) workgroup
        const float4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int idx = tid + 256 * u;
            const int r = idx >> 5, c = (idx & 31) * 4;
            if (r < rows) {
                const int64_t e = ((sq.b * a.T + t0 + r) * a.H + h) * DK + c;
                *reinterpret_cast<float4*>(a.dq + e) = z;
                *reinterpret_cast<float4*>(a.dk + e) = z;
                *reinterpret_cast<float4*>(a.dg + e) = z;
            }
        }
        if (tid < rows) a.dbeta[(sq.b * a.T + t0 + tid) * a.H + h] = 0.f;
    }
    // loads: 16 rows x 32 quads, two quads per thread
    Raw4<Tin> q[2], k[2], g[2];
    bool in[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int idx = tid + 256 * u;
        const int r = idx >> 5, c = (idx & 31) * 4;
        in[u] = r < rows;
        const int64_t e = ((sq.b * a.T + t0 + (in[u] ? r : 0)) * a.H + h) * DK + c;
        q[u].load(static_cast<const Tin*>(a.q), e);
        k[u].load(static_cast<const Tin*>(a.k), e);
        g[u].load(static_cast<const Tin*>(a.g), e);
    }
    const bool inb = (tid & (C - 1)) < rows;
    const float bt = load_elem(static_cast<const Tin*>(a.beta), (sq.b * a.T + t0 + (inb ? (tid & (C - 1)) : 0)) * a.H + h);
    if (a.status) {
        // the factored exponentials below need g in [-5, 0] (NaN fails too):
        // a wave that meets one outside counts it in status word 1
        bool bad = false;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = g[u].get(e);
                bad |= in[u] && !(x >= -5.f && x <= 0.f);
            }
        if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0)
            __hip_atomic_fetch_add(a.status + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int idx = tid + 256 * u;
        const int r = idx >> 5, c = (idx & 31) * 4;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            sm.G[r][c + v] = in[u] ? g[u].get(v) * kLog2e : 0.f;
            sm.Kp[r][c + v] = in[u] ? k[u].get(v) : 0.f;
            sm.Qp[r][c + v] = in[u] ? q[u].get(v) : 0.f;
        }
    }
    if (tid < C) sm.beta[tid] = inb ? bt : 0.f;
    __syncthreads();
    if (tid < DK) {
        float run = 0.f;
#pragma unroll
        for (int r = 0; r < C; ++r) {
            run += sm.G[r][tid];
            sm.G[r][tid] = run;
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int idx = tid + 256 * u;
        const int r = idx / DK, c = idx % DK;
        const float d = sm.G[r][c] - sm.G[kRef][c];
        const float k0 = sm.Kp[r][c];
        const float ep = __builtin_amdgcn_exp2f(d);
        sm.Kp[r][c] = ep * k0;
        sm.Qp[r][c] *= ep;
        sm.Km[r][c] = __builtin_amdgcn_exp2f(-d) * k0;
    }
    __syncthreads();
    float* mats = a.ws + chunk_bwd_slots(a.B, a.T, a.N, a.cu != nullptr) * (int64_t)a.H * DK * a.Dv +
                  (slot * a.H + h) * kMats;
    if (w < 2) {   // wave 0: KK = Kp Km^T (strict lower); wave 1: P = Qp Km^T (lower)
        const float (*X)[KP] = w == 0 ? sm.Kp : sm.Qp;
        f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll
        for (int ks = 0; ks < DK / 4; ks += 2) {
            a0 = mfma(X[l16][4 * ks + lg], sm.Km[l16][4 * ks + lg], a0);
            a1 = mfma(X[l16][4 * ks + 4 + lg], sm.Km[l16][4 * ks + 4 + lg], a1);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * lg + i, s = l16;
            const float v = a0[i] + a1[i];
            if (w == 0) {
                const float kk = s < r ? v : 0.f;
                sm.KK[r][s] = kk;
                mats[2 * C * C + r * C + s] = kk;
            } else {
                mats[C * C + r * C + s] = s <= r ? v : 0.f;
            }
        }
    }
    __syncthreads();
    if (tid < C) {   // T by forward substitution, column tid in registers
        const int i = tid;
        float tc[C];
#pragma unroll
        for (int r = 0; r < C; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int s = 0; s < r; ++s) acc += sm.KK[r][s] * tc[s];
            tc[r] = r < i ? 0.f : (r == i ? 1.f : -sm.beta[r] * acc);
        }
#pragma unroll
        for (int r = 0; r < C; ++r) mats[r * C + i] = tc[r];
    }
}

// ---- forward sweep: one chunk's operands, prepared by waves 4-7 ----------
// An operand set of the forward sweep: the scaled rows Kg and Kh, V, T,
// beta and e^Gamma_C of one chunk.
struct FwdSet {
    float (*Kg)[KP];
    float (*Kh)[KP];
    float (*V)[VP];
    float (*T)[CP];
    float* beta;
    float* EC;
};

// One chunk's inputs for the forward sweep, in the registers of the 256
// prep threads (p = 0..255): k and g quads p and p + 256 of the 16 x 32, the
// v quad p of the 16 x 16, T entry p and beta of row p % 16.
template <typename Tin, typename Tx>
struct FwdFetch {
    Raw4<Tin> k[2], g[2];
    Raw4<Tx> v;
    Raw1<Tin> beta;
    float t;
    bool in_qk[2], in_v, in_b;
};

template <typename Tin, typename Tx>
__device__ __forceinline__ void fwd_fetch(FwdFetch<Tin, Tx>& f, const BwdArgs& a, const SeqInfo& sq, int h,
                                          int64_t t0, int rows, int c0, const float* mats, int p) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int q = p + 256 * u, r = q >> 5, c = (q & 31) * 4;
        f.in_qk[u] = r < rows;
        const int64_t e = ((sq.b * a.T + t0 + (f.in_qk[u] ? r : 0)) * a.H + h) * DK + c;
        f.k[u].load(static_cast<const Tin*>(a.k), e);
        f.g[u].load(static_cast<const Tin*>(a.g), e);
    }
    {
        const int r = p >> 4, j = (p & 15) * 4;
        f.in_v = r < rows;
        const int64_t e = ((sq.b * a.T + t0 + (f.in_v ? r : 0)) * a.H + h) * (int64_t)a.Dv + c0 + j;
        f.v.load(static_cast<const Tx*>(a.v), e);
    }
    {
        const int r = p & (C - 1);
        f.in_b = r < rows;
        f.beta.load(static_cast<const Tin*>(a.beta), (sq.b * a.T + t0 + (f.in_b ? r : 0)) * a.H + h);
    }
    f.t = mats[p];   // T[p / C][p % C]
}

// raw k into Kg, the log2-scaled gate into G, v, T and beta (rows past the
// sequence end are zero tokens)
template <typename Tin, typename Tx>
__device__ __forceinline__ void fwd_commit(Smem& sm, const FwdFetch<Tin, Tx>& f, const FwdSet& s, int p) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int q = p + 256 * u, r = q >> 5, c = (q & 31) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s.Kg[r][c + e] = f.in_qk[u] ? f.k[u].get(e) : 0.f;
            sm.G[r][c + e] = f.in_qk[u] ? f.g[u].get(e) * kLog2e : 0.f;
        }
    }
    {
        const int r = p >> 4, j = (p & 15) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) s.V[r][j + e] = f.in_v ? f.v.get(e) : 0.f;
    }
    s.T[p / C][p % C] = f.t;
    if (p < C) s.beta[p] = f.in_b ? f.beta.get() : 0.f;
}

// Gamma (the in-chunk cumulative log2 decay) per channel and e^Gamma_C
__device__ __forceinline__ void fwd_gamma(Smem& sm, const FwdSet& s, int p) {
    if (p < DK) {
        float run = 0.f;
#pragma unroll
        for (int r = 0; r < C; ++r) {
            run += sm.G[r][p];
            sm.G[r][p] = run;
        }
        s.EC[p] = __builtin_amdgcn_exp2f(run);
    }
}

// Kg = e^Gamma k and Kh = e^(Gamma_C - Gamma) k
__device__ __forceinline__ void fwd_scale(Smem& sm, const FwdSet& s, int p) {
#pragma unroll
    for (int u = 0; u < C * DK / 256; ++u) {
        const int idx = p + 256 * u;
        const int r = idx / DK, c = idx % DK;
        const float gr = sm.G[r][c];
        const float k = s.Kg[r][c];
        s.Kg[r][c] = __builtin_amdgcn_exp2f(gr) * k;
        s.Kh[r][c] = __builtin_amdgcn_exp2f(sm.G[C - 1][c] - gr) * k;
    }
}

// Tin: q, k, g and beta; Tx: v and dO (bf16 v and dO with float32 q, k, g
// and beta come from the backward through the prologue, which widens only
// what it computes).
template <typename Tin, typename Tx>
__global__ __launch_bounds__(NT) void chunk_bwd_mfma_kernel(BwdArgs a) {
    __shared__ __attribute__((aligned(16))) Smem sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, lg = lane >> 4;
    const int nvt = a.Dv / BV;
    const bool atomic = nvt > 1;
    const int vt = blockIdx.x % nvt, unit = blockIdx.x / nvt;
    const int n = unit / a.H, h = unit % a.H;
    const int H = a.H, Dv = a.Dv, c0 = vt * BV;
    const float scale = a.scale;
    const SeqInfo sq = seq_info(a, n);
    const int64_t sbase = ((int64_t)n * H + h) * DK * (int64_t)Dv;
    const int64_t slot_stride = (int64_t)H * DK * Dv;
    const int64_t nch = (sq.len + C - 1) / C;
    const int cw = 16 * w;   // this wave's state rows / channel tile
    const float* mats0 = a.ws + chunk_bwd_slots(a.B, a.T, a.N, a.cu != nullptr) * slot_stride;
    auto mats_of = [&](int64_t ch) { return mats0 + ((sq.slot0 + ch) * H + h) * kMats; };
    auto state_of = [&](int64_t ch) { return a.ws + (sq.slot0 + ch) * slot_stride + (int64_t)h * DK * Dv + c0; };
    Fetch<Tin, Tx> f;

    // ---------------- forward sweep: chunk entry states ----------------
    // Waves 0-3 carry the state (wave w: rows 32w..32w+31, MFMA result
    // layout) through the chunks and store each chunk's entry state; waves
    // 4-7 meanwhile load, commit and scale the next chunk into the other of
    // two operand sets (the second set lives in arrays only the reverse
    // sweep uses). Three barriers per chunk, each the end of a phase of both
    // roles:
    //   1. state rows to LDS                   | commit chunk c+1, fetch c+3
    //   2. W = V - Kg S and U = T Diag(beta) W, one 16-column tile per wave
    //                                         | Gamma of chunk c+1, e^Gamma_C
    //   3. S <- Diag(e^Gamma_C) S + Kh^T U, then the entry state from LDS to
    //      the workspace                      | Kg, Kh of chunk c+1
    const bool chain = w < 4;
    const int ptid = tid - 256;   // prep threads: 0..255
    FwdSet set0{sm.Kg, sm.Kh, sm.dUW, sm.T, sm.beta, sm.EC};
    FwdSet set1{sm.Qp, sm.Kp, sm.dO, sm.P, sm.dbp, &sm.dS[0][0]};
    f32x4 st[2][4];
    if (chain) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    st[rt][t][i] = a.s0 ? a.s0[sbase + (int64_t)(32 * w + 16 * rt + 4 * lg + i) * Dv + c0 + 16 * t + l16]
                                        : 0.f;
    }
    auto rows_of = [&](int64_t ch) { return (int)min<int64_t>(C, sq.len - ch * C); };
    // Chunk ch's inputs into a prep register set. Past the last chunk the
    // fetch re-reads the last chunk with no rows: such a chunk is all zero
    // tokens, an exact identity step of the state.
    auto fetch_fwd = [&](FwdFetch<Tin, Tx>& dst, int64_t ch) {
        const int64_t cc = ch < nch ? ch : nch - 1;
        fwd_fetch<Tin, Tx>(dst, a, sq, h, sq.bos + cc * C, ch < nch ? rows_of(ch) : 0, c0, mats_of(cc), ptid);
    };
    FwdFetch<Tin, Tx> fa, fb;
    if (nch > 0) {
        // chunk 0 prepared before the loop; chunks 1 and 2 in flight
        if (!chain) {
            fetch_fwd(fa, 0);
            fetch_fwd(fb, 1);
            fwd_commit(sm, fa, set0, ptid);
            fetch_fwd(fa, 2);
        }
        __syncthreads();
        if (!chain) fwd_gamma(sm, set0, ptid);
        __syncthreads();
        if (!chain) fwd_scale(sm, set0, ptid);
        __syncthreads();
    }
    // chunk ch with its operands in `cur`; the prep waves commit chunk ch+1
    // from `fn` into `nxt` and refill `fn` with chunk ch+3
    auto fwd_chunk = [&](int64_t ch, const FwdSet& cur, const FwdSet& nxt, FwdFetch<Tin, Tx>& fn) {
        if (chain) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) sm.S[32 * w + 16 * rt + 4 * lg + i][16 * t + l16] = st[rt][t][i];
        } else {
            fwd_commit(sm, fn, nxt, ptid);
            fetch_fwd(fn, ch + 3);
        }
        __syncthreads();
        if (chain) {
            // W = V - Kg S, columns 16w..16w+15, then U for the same columns
            f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll 8
            for (int ks = 0; ks < DK / 4; ks += 2) {
                a0 = mfma(cur.Kg[l16][4 * ks + lg], sm.S[4 * ks + lg][16 * w + l16], a0);
                a1 = mfma(cur.Kg[l16][4 * ks + 4 + lg], sm.S[4 * ks + 4 + lg][16 * w + l16], a1);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * lg + i, j = 16 * w + l16;
                sm.W[r][j] = cur.V[r][j] - (a0[i] + a1[i]);
            }
            f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < C / 4; ++ks) {
                const int r = 4 * ks + lg;
                u = mfma(cur.T[l16][r], cur.beta[r] * sm.W[r][16 * w + l16], u);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.U[4 * lg + i][16 * w + l16] = u[i];
        } else {
            fwd_gamma(sm, nxt, ptid);
        }
        __syncthreads();
        if (chain) {
            // S <- Diag(e^Gamma_C) S + Kh^T U, rows 32w..32w+31
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const int cw2 = 32 * w + 16 * rt;
                float ak[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) ak[ks] = cur.Kh[4 * ks + lg][cw2 + l16];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    f32x4 acc;
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] = cur.EC[cw2 + 4 * lg + i] * st[rt][t][i];
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) acc = mfma(ak[ks], sm.U[4 * ks + lg][16 * t + l16], acc);
                    st[rt][t] = acc;
                }
            }
            // the entry state (still in sm.S) to the workspace, in 16-byte
            // pieces of this wave's rows: here, after the products, they neither
            // delay the products' LDS reads nor queue ahead of the prep waves'
            // loads in phase 1
            if (ch < nch) {
                float* ws = state_of(ch);
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int q = lane + 64 * u, c = 32 * w + (q >> 4), j = (q & 15) * 4;
                    *reinterpret_cast<float4*>(ws + (int64_t)c * Dv + j) = *reinterpret_cast<const float4*>(&sm.S[c][j]);
                }
            }
        } else {
            fwd_scale(sm, nxt, ptid);
        }
        __syncthreads();
    };
    for (int64_t ch = 0; ch < nch; ch += 2) {
        fwd_chunk(ch, set0, set1, fb);
        fwd_chunk(ch + 1, set1, set0, fa);
    }
    // the entry states stored above are read below by other waves
    __syncthreads();

    // ---------------- backward sweep ----------------
    f32x4 ds[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            ds[t][i] = a.d_final ? a.d_final[sbase + (int64_t)(cw + 4 * lg + i) * Dv + c0 + 16 * t + l16] : 0.f;
    for (int64_t ch = nch - 1; ch >= 0; --ch) {
        const int64_t t0 = sq.bos + ch * C;
        const int rows = rows_of(ch);
        fetch_chunk<Tin, Tx>(f, a, sq, h, t0, rows, c0, true, state_of(ch), mats_of(ch));
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.dS[cw + 4 * lg + i][16 * t + l16] = ds[t][i];
        // With float32 q, k and g (twice the bytes of bf16) the rest of the
        // chunk is committed after the scaling phase, which none of it
        // feeds, so its loads keep arriving meanwhile: -2% at B=1 T=4096
        // H=96. With bf16 inputs committing it all up front measured 1% faster.
        commit_qkg<Tin, Tx>(sm, f, true);
        if constexpr (sizeof(Tin) == 2) commit_rest<Tin, Tx>(sm, f, true);
        __syncthreads();
        chunk_scale(sm, true);
        if constexpr (sizeof(Tin) == 4) commit_rest<Tin, Tx>(sm, f, true);
        __syncthreads();
        // W = V - Kg S (waves 0-3);  dU = scale P^T dO + Kh dS (waves 4-7)
        if (w < 4) {
            w_tile(sm, w, l16, lg);
        } else {
            const int t = w - 4;
            f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, ap = a0;
#pragma unroll 8
            for (int ks = 0; ks < DK / 4; ks += 2) {
                a0 = mfma(sm.Kh[l16][4 * ks + lg], sm.dS[4 * ks + lg][16 * t + l16], a0);
                a1 = mfma(sm.Kh[l16][4 * ks + 4 + lg], sm.dS[4 * ks + 4 + lg][16 * t + l16], a1);
            }
#pragma unroll
            for (int ks = 0; ks < C / 4; ++ks)
                ap = mfma(sm.P[4 * ks + lg][l16], sm.dO[4 * ks + lg][16 * t + l16], ap);
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.dUW[4 * lg + i][16 * t + l16] = a0[i] + a1[i] + scale * ap[i];
        }
        __syncthreads();
        // U = T Diag(beta) W (waves 0-3);  dY = T^T dU (waves 4-7)
        if (w < 4) {
            u_tile(sm, w, l16, lg);
        } else {
            const int t = w - 4;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < C / 4; ++ks)
                acc = mfma(sm.T[4 * ks + lg][l16], sm.dUW[4 * ks + lg][16 * t + l16], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.dY[4 * lg + i][16 * t + l16] = acc[i];
        }
        __syncthreads();
        // dP = scale dO U^T (wave 0);  dKK = -Diag(beta) dY U^T and its part of
        // dbeta (wave 1);  dY_r . W_r (wave 2);  dW = Diag(beta) dY = dV (all)
        if (w == 0) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < BV / 4; ++ks)
                acc = mfma(sm.dO[l16][4 * ks + lg], sm.U[l16][4 * ks + lg], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * lg + i;
                sm.dP[r][l16] = l16 <= r ? scale * acc[i] : 0.f;
            }
        } else if (w == 1) {
            f32x4 am = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < BV / 4; ++ks) am = mfma(sm.dY[l16][4 * ks + lg], sm.U[l16][4 * ks + lg], am);
            // sum_s dM[r][s] KK[r][s]
            float part[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * lg + i, s = l16;
                const float dm = s < r ? -am[i] : 0.f;
                sm.dKK[r][s] = sm.beta[r] * dm;
                part[i] = row16_sum(dm * sm.KK[r][s]);
            }
            if (l16 == 15) {
#pragma unroll
                for (int i = 0; i < 4; ++i) sm.dbp[4 * lg + i] = part[i];
            }
        } else if (w == 2) {
            // dY_r . W_r: the diagonal of dY W^T
            f32x4 ax = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < BV / 4; ++ks) ax = mfma(sm.dY[l16][4 * ks + lg], sm.W[l16][4 * ks + lg], ax);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (l16 == 4 * lg + i) sm.xd[l16] = ax[i];
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int idx = tid + NT * u;
            const int r = idx / BV, j = idx % BV;
            const float dw = sm.beta[r] * sm.dY[r][j];
            sm.dUW[r][j] = dw;
            if (r < rows) a.dv[((sq.b * a.T + t0 + r) * H + h) * (int64_t)Dv + c0 + j] = dw;
        }
        __syncthreads();
        if (tid < C && tid < rows)   // dbeta_r = dY_r . W_r + sum_s dM[r][s] KK[r][s]
            add_out(a.dbeta + (sq.b * a.T + t0 + tid) * H + h, sm.xd[tid] + sm.dbp[tid], atomic);
        // Channel tile cw..cw+15 of this wave: dense terms, pair terms, dq,
        // dk, dg, then the state gradient's rows cw..cw+15.
        {
            const int c = cw + l16;
            f32x4 ao = {0.f, 0.f, 0.f, 0.f}, aw = ao, ad = ao;
#pragma unroll 4
            for (int ks = 0; ks < BV / 4; ++ks) {
                const int j = 4 * ks + lg;
                const float sv = sm.S[c][j];
                ao = mfma(sm.dO[l16][j], sv, ao);
                aw = mfma(sm.dUW[l16][j], sv, aw);
                ad = mfma(sm.U[l16][j], sm.dS[c][j], ad);
            }
            // pair terms, factored through the reference row:
            //   Aq = dP Km, Akr = dKK Km, Aks = dP^T Qp + dKK^T Kp
            f32x4 aq = {0.f, 0.f, 0.f, 0.f}, akr = aq, aks = aq;
#pragma unroll
            for (int ks = 0; ks < C / 4; ++ks) {
                const int s = 4 * ks + lg;
                const float km = sm.Km[s][c];
                aq = mfma(sm.dP[l16][s], km, aq);
                akr = mfma(sm.dKK[l16][s], km, akr);
                aks = mfma(sm.dP[s][l16], sm.Qp[s][c], aks);
                aks = mfma(sm.dKK[s][l16], sm.Kp[s][c], aks);
            }
            const float gC = sm.G[C - 1][c], gref = sm.G[kRef][c];
            float dG[4], kh_ad = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * lg + i;
                const float gr = sm.G[r][c];
                const float eg = __builtin_amdgcn_exp2f(gr);
                const float eh = __builtin_amdgcn_exp2f(gC - gr);
                const float ep = __builtin_amdgcn_exp2f(gr - gref);
                const float em = __builtin_amdgcn_exp2f(gref - gr);
                const float qh = sm.Qh[r][c], kg = sm.Kg[r][c], kh = sm.Kh[r][c];
                const float dq = ep * aq[i] + eg * scale * ao[i];
                const float dk = ep * akr[i] + em * aks[i] - eg * aw[i] + eh * ad[i];
                dG[i] = sm.Qp[r][c] * aq[i] + sm.Kp[r][c] * akr[i] - sm.Km[r][c] * aks[i] + qh * scale * ao[i] -
                        kg * aw[i] - kh * ad[i];
                kh_ad += kh * ad[i];
                if (r < rows) {
                    const int64_t e2 = ((sq.b * a.T + t0 + r) * H + h) * DK + c;
                    add_out(a.dq + e2, dq, atomic);
                    add_out(a.dk + e2, dk, atomic);
                }
            }
            // Gamma_C's gradient: sum_r Kh*ad over the 16 rows + e^Gamma_C sum_j dS S
            float sds = 0.f;
#pragma unroll
            for (int m = 0; m < BV / 4; ++m) sds += sm.dS[c][lg + 4 * m] * sm.S[c][lg + 4 * m];
            float gsum = kh_ad + sm.EC[c] * sds;
            gsum += __shfl_xor(gsum, 16, 64);
            gsum += __shfl_xor(gsum, 32, 64);
            // dg = reverse cumulative sum of dGamma over the chunk, plus gsum
            const float s3 = dG[3], s2 = dG[2] + s3, s1 = dG[1] + s2, s0v = dG[0] + s1;
            const float t1 = __shfl(s0v, l16 + 16, 64), t2 = __shfl(s0v, l16 + 32, 64),
                        t3 = __shfl(s0v, l16 + 48, 64);
            const float above = (lg < 1 ? t1 : 0.f) + (lg < 2 ? t2 : 0.f) + (lg < 3 ? t3 : 0.f) + gsum;
            const float sfx[4] = {s0v, s1, s2, s3};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * lg + i;
                if (r < rows) add_out(a.dg + ((sq.b * a.T + t0 + r) * H + h) * DK + c, sfx[i] + above, atomic);
            }
            // dS <- Diag(e^Gamma_C) dS + scale Qh^T dO - Kg^T dW   (rows cw..cw+15)
            float aqh[4], akg[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                aqh[ks] = scale * sm.Qh[4 * ks + lg][cw + l16];
                akg[ks] = -sm.Kg[4 * ks + lg][cw + l16];
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                f32x4 acc;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = sm.EC[cw + 4 * lg + i] * ds[t][i];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    acc = mfma(aqh[ks], sm.dO[4 * ks + lg][16 * t + l16], acc);
                    acc = mfma(akg[ks], sm.dUW[4 * ks + lg][16 * t + l16], acc);
                }
                ds[t] = acc;
            }
        }
        __syncthreads();
    }
    if (a.d_s0) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a.d_s0[sbase + (int64_t)(cw + 4 * lg + i) * Dv + c0 + 16 * t + l16] = ds[t][i];
    }
}

}  // namespace mf
}  // namespace


bool chunk_bwd_mfma_supported(const BwdArgs& a);

hipError_t launch_chunk_bwd(const BwdArgs& args, hipStream_t s) {
    const int nvt = args.Dv / (chunk_bwd_mfma_supported(args) ? mf::BV : vbwd_bv(args.Dv));
    BwdArgs a = args;
    // the matrix-core path zeroes the atomically summed gradients in its T/P/KK kernel
    a.zero_grads = nvt > 1 && chunk_bwd_mfma_supported(a);
    if (nvt > 1 && !a.zero_grads) {
        const int64_t rows = (int64_t)a.B * a.T * a.H;
        hipError_t e;
        if ((e = zero_fill(a.dq, rows * a.Dk, s)) != hipSuccess) return e;
        if ((e = zero_fill(a.dk, rows * a.Dk, s)) != hipSuccess) return e;
        if ((e = zero_fill(a.dg, rows * a.Dk, s)) != hipSuccess) return e;
        if ((e = zero_fill(a.dbeta, rows, s)) != hipSuccess) return e;
    }
    if (chunk_bwd_mfma_supported(a)) {
        const int64_t grid = (int64_t)a.N * a.H * (a.Dv / mf::BV);
        const int64_t slots = chunk_bwd_slots(a.B, a.T, a.N, a.cu != nullptr);
        if (grid == 0) return hipSuccess;
        if (slots > 0) {
            const dim3 mg((unsigned)slots, (unsigned)a.H);
            if (a.bf16)
                mf::chunk_mats_kernel<__bf16><<<mg, dim3(256), 0, s>>>(a);
            else
                mf::chunk_mats_kernel<float><<<mg, dim3(256), 0, s>>>(a);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        if (a.bf16)
            mf::chunk_bwd_mfma_kernel<__bf16, __bf16><<<dim3((unsigned)grid), dim3(mf::NT), 0, s>>>(a);
        else if (a.x_bf16)
            mf::chunk_bwd_mfma_kernel<float, __bf16><<<dim3((unsigned)grid), dim3(mf::NT), 0, s>>>(a);
        else
            mf::chunk_bwd_mfma_kernel<float, float><<<dim3((unsigned)grid), dim3(mf::NT), 0, s>>>(a);
        return hipGetLastError();
    }
    if (a.x_bf16) return hipErrorInvalidValue;   // mixed input types: matrix-core path only
    return a.bf16 ? launch_dtype<__bf16>(a, s) : launch_dtype<float>(a, s);
}

bool chunk_bwd_mfma_supported(const BwdArgs& a) {
    return a.Dk == 128 && (a.Dv == 64 || a.Dv == 128) && a.g_ge_m5;
}

}  // namespace kda
