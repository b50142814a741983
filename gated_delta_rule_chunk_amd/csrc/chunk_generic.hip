// Chunkwise KDA forward in float32 arithmetic: the general path for
// every supported (dtype, Dk, Dv, chunk) combination that the bf16
// matrix-core kernel does not cover.
//
// One workgroup owns one (sequence, head, slice of BV columns of d_v) and
// walks the sequence chunk by chunk, carrying the float32 state slice in LDS.
// Per chunk of C rows with entry state S (Gamma = in-chunk cumulative
// log-decay per channel, gamma = exp(Gamma)):
//   M[r][i] = beta_r * sum_c k_rc k_ic exp(Gamma_rc - Gamma_ic)   (i < r)
//   P[r][i] =          sum_c q_rc k_ic exp(Gamma_rc - Gamma_ic)   (i <= r)
//   (I + M) U = Diag(beta) (V - (gamma*K) S)         forward substitution
//   O = scale * ((gamma*Q) S + P U)
//   S <- Diag(gamma_C) S + (exp(Gamma_C - Gamma) * K)^T U
// This is the WY/UT-transform chunk form of the gated delta rule with a
// per-channel decay. The grams take the factored form (gamma*K)(K/gamma)^T,
// (gamma*Q)(K/gamma)^T when every channel's cumulative decay in the chunk
// stays within [-80, 80] (so gamma and 1/gamma are finite); a chunk with
// stronger decay takes every pair's exponential of its own difference instead
// (non-positive for g <= 0), so no range precondition on g is needed on this
// path.
//
// With 16-row chunks the grams (factored form), the two products with the
// state, P U and the state update run on the matrix cores as float32 16x16x4
// products; longer chunks run them on the vector ALUs as register tiles (4
// output columns per thread, 4 x 4 for the update). The next chunk's inputs
// are loaded into registers while the current one is computed.
//
// With the prologue (ChunkArgs::prologue), rows are loaded as raw projections
// and turned into the recurrence's inputs on the way into LDS:
//   g = lb * sigmoid(exp(A_log[c]) * (logit + dt_bias[h][c])), beta =
//   sigmoid(logit), q and k scaled to x / sqrt(|x|^2 + eps) per row.
// Rows past a sequence's end keep g = beta = 0 and zero q, k.
#include "device_common.hpp"
#include "launchers.hpp"

namespace kda {
namespace {

constexpr int kGenThreads = 512;
constexpr float kMaxChunkDecay = 80.f;   // factored grams while every -Gamma_C <= this

// Value columns per workgroup: 64 (or all of d_v) for 16- and 32-row chunks;
// 16 for 64-row chunks, whose K, Q and Gamma tiles fill most of the LDS.
constexpr int gen_bv(int C, int DV) { return C == 64 ? 16 : (DV < 64 ? DV : 64); }

// The inputs of one chunk in registers, loaded ahead (element e of thread
// tid: row/channel index tid + NT e of the C x DK tiles, and of C x BV for v).
template <int DK, int C, int BV, typename Tin>
struct GenRegs {
    static constexpr int kNK = (C * DK + kGenThreads - 1) / kGenThreads;
    static constexpr int kNV = (C * BV + kGenThreads - 1) / kGenThreads;
    float q[kNK], k[kNK], g[kNK], v[kNV];
    float beta;
};

template <int DK, int C, int BV, typename Tin>
__device__ __forceinline__ void gen_load(GenRegs<DK, C, BV, Tin>& R, const ChunkArgs& a, int64_t tok0, int rows,
                                         int h, int c0) {
    const Tin* q = static_cast<const Tin*>(a.q);
    const Tin* k = static_cast<const Tin*>(a.k);
    const Tin* g = static_cast<const Tin*>(a.g);
    const Tin* v = static_cast<const Tin*>(a.v);
    const Tin* beta = static_cast<const Tin*>(a.beta);
    const int tid = threadIdx.x;
#pragma unroll
    for (int e = 0; e < R.kNK; ++e) {
        const int idx = tid + kGenThreads * e;
        const int r = idx / DK, c = idx % DK;
        const bool in = idx < C * DK && r < rows;
        const int64_t off = ((tok0 + r) * a.H + h) * DK + c;
        R.q[e] = in ? load_elem(q, off) : 0.f;
        R.k[e] = in ? load_elem(k, off) : 0.f;
        R.g[e] = in ? load_elem(g, off) : 0.f;
    }
#pragma unroll
    for (int e = 0; e < R.kNV; ++e) {
        const int idx = tid + kGenThreads * e;
        const int r = idx / BV, j = idx % BV;
        const bool in = idx < C * BV && r < rows && v;
        R.v[e] = in ? load_elem(v, ((tok0 + r) * a.H + h) * a.Dv + c0 + j) : 0.f;
    }
    R.beta = tid < rows ? load_elem(beta, (tok0 + tid) * a.H + h) : 0.f;
}

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

template <int DK, int C, int BV, typename Tin>
__global__ __launch_bounds__(kGenThreads) void chunk_generic_kernel(ChunkArgs a) {
    constexpr int NT = kGenThreads;
    constexpr int DKP = DK + 4;     // row stride of the C x DK tiles (16-byte rows; row r starts at bank 4r)
    constexpr int BVP = BV + 4;     // row stride of the C x BV and DK x BV tiles (16-byte rows)
    static_assert(C <= NT && DK <= NT, "one thread per row / channel");
    __shared__ __attribute__((aligned(16))) float sK[C][DKP];
    __shared__ __attribute__((aligned(16))) float sQ[C][DKP];
    __shared__ __attribute__((aligned(16))) float sG[C][DKP];
    __shared__ float sA[C][C + 1];
    __shared__ float sP[C][C + 1];
    __shared__ __attribute__((aligned(16))) float sV[C][BVP];
    __shared__ __attribute__((aligned(16))) float sU[C][BVP];
    __shared__ __attribute__((aligned(16))) float sS[DK][BVP];
    __shared__ float sBeta[C];
    __shared__ float sGn[DK];
    __shared__ float sEd[DK];     // exp(Gamma_C): the chunk's decay of each state row
    __shared__ float sAe[DK];     // prologue: exp(A_log)
    __shared__ float sDb[DK];     // prologue: dt_bias of this head

    Tin* o = static_cast<Tin*>(a.o);
    const int tid = threadIdx.x;
    // 16-row chunks run their dense products on the matrix cores (f32
    // 16x16x4: float32 operands, float32 sums). Operand layouts, lane l with
    // l16 = l % 16, lg = l / 16: A[m][k] at m = l16, k = lg; B[k][n] at k = lg,
    // n = l16; result register i holds D[4 lg + i][l16].
    constexpr bool kMfma = C == 16;
    constexpr int NTL = BV / 16;    // 16-column tiles of the slice
    const int wave = tid / 64, l16 = tid % 16, lg = (tid % 64) / 16;
    const int mp = wave / NTL, mt = wave % NTL;   // rhs/output: product (0: K, 1: Q) and column tile of this wave
    const int nvt = a.Dv / BV;
    const int unit = blockIdx.x / nvt;
    const int vt = blockIdx.x % nvt;
    const int n = unit / a.H;
    const int h = unit % a.H;
    const int H = a.H, Dv = a.Dv;
    int64_t bos, len, b;
    if (a.cu) {
        bos = a.cu[n];
        len = (int64_t)a.cu[n + 1] - bos;
        b = 0;
    } else {
        bos = 0;
        len = a.T;
        b = n;
    }
    const int c0 = vt * BV;
    const int64_t state_base = ((int64_t)n * H + h) * DK * (int64_t)Dv;

    for (int idx = tid; idx < DK * BV; idx += NT) {
        const int r = idx / BV, c = idx % BV;
        sS[r][c] = a.s0 ? a.s0[state_base + (int64_t)r * Dv + c0 + c] : 0.f;
    }
    if (a.prologue) {
        for (int c = tid; c < DK; c += NT) {
            sAe[c] = expf(a.A_log[c]);
            sDb[c] = a.dt_bias[h * DK + c];
        }
    }
    __syncthreads();

    GenRegs<DK, C, BV, Tin> R;
    if (len > 0) gen_load(R, a, b * (int64_t)a.T + bos, (int)(len < C ? len : C), h, c0);

    for (int64_t cs = 0; cs < len; cs += C) {
        const int rows = (int)((len - cs) < C ? (len - cs) : C);
        const int64_t tok0 = b * (int64_t)a.T + bos + cs;  // token index of chunk row 0
        // commit this chunk's inputs (the previous chunk's last reads of these
        // tiles are behind the barrier that ended it)
#pragma unroll
        for (int e = 0; e < R.kNK; ++e) {
            const int idx = tid + NT * e;
            if (idx < C * DK) {
                const int r = idx / DK, c = idx % DK;
                float gv = R.g[e];
                if (a.prologue && r < rows) gv = a.gate_lb / (1.f + expf(-sAe[c] * (gv + sDb[c])));
                sQ[r][c] = R.q[e];
                sK[r][c] = R.k[e];
                sG[r][c] = gv;
            }
        }
#pragma unroll
        for (int e = 0; e < R.kNV; ++e) {
            const int idx = tid + NT * e;
            if (idx < C * BV) sV[idx / BV][idx % BV] = R.v[e];
        }
        if (tid < C) sBeta[tid] = a.prologue && tid < rows ? 1.f / (1.f + expf(-R.beta)) : R.beta;
        // the next chunk's loads, in flight while this one is computed
        if (cs + C < len) {
            const int64_t rem = len - cs - C;
            gen_load(R, a, tok0 + C, (int)(rem < C ? rem : C), h, c0);
        }
        __syncthreads();
        if (a.prologue) {
            // q and k rows to unit length (eps > 0: zero rows stay zero)
            for (int idx = tid; idx < 2 * C; idx += NT) {
                f32x4* row = reinterpret_cast<f32x4*>(idx < C ? sQ[idx] : sK[idx - C]);
                float ss = 0.f;
                for (int c4 = 0; c4 < DK / 4; ++c4) {
                    const f32x4 x = row[c4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) ss += x[u] * x[u];
                }
                const float rs = 1.f / sqrtf(ss + a.l2_eps);
                for (int c4 = 0; c4 < DK / 4; ++c4) row[c4] *= rs;
            }
            __syncthreads();
        }

        // in-chunk cumulative log-decay, one channel per thread; a chunk whose
        // cumulative decay leaves [-80, 80] on some channel (or is not finite)
        // takes the pairwise grams
        bool steep = false;
        if (tid < DK) {
            float acc = 0.f, lo = 0.f, hi = 0.f;
            for (int r = 0; r < C; ++r) {
                acc += sG[r][tid];
                sG[r][tid] = acc;
                lo = fminf(lo, acc);
                hi = fmaxf(hi, acc);
            }
            sGn[tid] = acc;
            sEd[tid] = expf(acc);
            steep = !(lo >= -kMaxChunkDecay && hi <= kMaxChunkDecay && acc == acc);
        }
        steep = __syncthreads_or(steep);

        if (steep) {
            // pairwise: every exponential of a non-positive difference
            for (int idx = tid; idx < C * C; idx += NT) {
                const int r = idx / C, i = idx % C;
                float am = 0.f, pm = 0.f;
                if (i <= r) {
                    for (int c = 0; c < DK; c += 4) {
                        const f32x4 kb = ld4(&sK[i][c]), gi = ld4(&sG[i][c]), gr = ld4(&sG[r][c]);
                        const f32x4 kr = ld4(&sK[r][c]), qr = ld4(&sQ[r][c]);
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const float ki = kb[u] * expf(gr[u] - gi[u]);
                            am += kr[u] * ki;
                            pm += qr[u] * ki;
                        }
                    }
                }
                sA[r][i] = (i < r) ? sBeta[r] * am : 0.f;
                sP[r][i] = pm;
            }
            __syncthreads();
            // gamma*Q into sQ, gamma*K into sG, exp(Gamma_C - Gamma)*K into sK
            for (int idx = tid; idx < C * DK; idx += NT) {
                const int r = idx / DK, c = idx % DK;
                const float gv = sG[r][c];
                const float kv = sK[r][c];
                const float eg = expf(gv);
                sQ[r][c] *= eg;
                sG[r][c] = kv * eg;
                sK[r][c] = kv * expf(sGn[c] - gv);
            }
            __syncthreads();
        } else {
            // gamma*Q into sQ, gamma*K into sG, K/gamma into sK
            for (int idx = tid; idx < C * DK; idx += NT) {
                const int r = idx / DK, c = idx % DK;
                const float eg = expf(sG[r][c]);
                const float kv = sK[r][c];
                sQ[r][c] *= eg;
                sG[r][c] = kv * eg;
                sK[r][c] = kv * __builtin_amdgcn_rcpf(eg);
            }
            __syncthreads();
            if constexpr (kMfma) {
                // waves 0 and 1: (gamma*K)(K/gamma)^T and (gamma*Q)(K/gamma)^T
                if (wave < 2) {
                    const float(*X)[DKP] = wave ? sQ : sG;
                    f32x4 gm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
                    for (int s4 = 0; s4 < DK; s4 += 4)
                        gm = __builtin_amdgcn_mfma_f32_16x16x4f32(X[l16][s4 + lg], sK[l16][s4 + lg], gm, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = 4 * lg + i;
                        if (wave == 0)
                            sA[m][l16] = l16 < m ? sBeta[m] * gm[i] : 0.f;
                        else
                            sP[m][l16] = l16 <= m ? gm[i] : 0.f;
                    }
                }
            } else {
                for (int idx = tid; idx < C * C; idx += NT) {
                    const int r = idx / C, i = idx % C;
                    float am = 0.f, pm = 0.f;
                    if (i <= r) {
#pragma unroll 4
                        for (int c = 0; c < DK; c += 4) {
                            const f32x4 kb = ld4(&sK[i][c]), gr = ld4(&sG[r][c]), qr = ld4(&sQ[r][c]);
#pragma unroll
                            for (int u = 0; u < 4; ++u) {
                                am += gr[u] * kb[u];
                                pm += qr[u] * kb[u];
                            }
                        }
                    }
                    sA[r][i] = (i < r) ? sBeta[r] * am : 0.f;
                    sP[r][i] = pm;
                }
            }
            __syncthreads();

            // K/gamma to exp(Gamma_C - Gamma)*K for the state update
            for (int idx = tid; idx < C * DK; idx += NT) {
                const int r = idx / DK, c = idx % DK;
                sK[r][c] *= sEd[c];
            }
        }

        // right-hand side Diag(beta)(V - (gamma*K) S), and the output's
        // (gamma*Q) S kept in registers. 16-row chunks: on the matrix cores
        // (f32 16x16x4, float32 operands and sums), wave w < 2 BV/16 owning one
        // 16 x 16 tile of one of the two products; longer chunks: 4 columns
        // per thread on the vector ALUs, one pass over S.
        f32x4 macc = {0.f, 0.f, 0.f, 0.f};
        constexpr int kRT = kMfma ? 1 : (C * (BV / 4) + NT - 1) / NT;
        f32x4 qs[kRT];
        if constexpr (kMfma) {
            if (wave < 2 * NTL) {
                const float(*A)[DKP] = mp ? sQ : sG;
#pragma unroll 8
                for (int s4 = 0; s4 < DK; s4 += 4)
                    macc = __builtin_amdgcn_mfma_f32_16x16x4f32(A[l16][s4 + lg], sS[s4 + lg][16 * mt + l16], macc, 0,
                                                                0, 0);
                if (mp == 0) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = 4 * lg + i, n = 16 * mt + l16;
                        sU[m][n] = sBeta[m] * (sV[m][n] - macc[i]);
                    }
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < kRT; ++e) {
                const int idx = tid + NT * e;
                if (idx < C * (BV / 4)) {
                    const int r = idx / (BV / 4), j = 4 * (idx % (BV / 4));
                    f32x4 y = {0.f, 0.f, 0.f, 0.f}, z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
                    for (int c = 0; c < DK; c += 4) {
                        const f32x4 gr = ld4(&sG[r][c]), qr = ld4(&sQ[r][c]);
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const f32x4 sv = ld4(&sS[c + u][j]);
                            y += gr[u] * sv;
                            z += qr[u] * sv;
                        }
                    }
                    qs[e] = z;
                    const f32x4 vv = *reinterpret_cast<const f32x4*>(&sV[r][j]);
                    *reinterpret_cast<f32x4*>(&sU[r][j]) = sBeta[r] * (vv - y);
                }
            }
        }
        __syncthreads();

        // (I + M) U = rhs by blocked forward substitution over 16-row blocks:
        // each diagonal block is solved with its columns in registers (one
        // column per thread), then the rows below subtract that block's terms
        // in parallel. Every row still subtracts its terms in ascending order,
        // as the plain substitution does. Rows past the sequence's end have
        // zero rhs and zero M rows, so they stay zero.
#pragma unroll
        for (int b0 = 0; b0 < C; b0 += 16) {
            for (int j = tid; j < BV; j += NT) {
                float u[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) u[r] = sU[b0 + r][j];
#pragma unroll
                for (int r = 1; r < 16; ++r) {
                    float acc = u[r];
#pragma unroll
                    for (int i = 0; i < r; ++i) acc -= sA[b0 + r][b0 + i] * u[i];
                    u[r] = acc;
                }
#pragma unroll
                for (int r = 1; r < 16; ++r) sU[b0 + r][j] = u[r];
            }
            __syncthreads();
            if (b0 + 16 < C) {
                for (int idx = tid; idx < (C - b0 - 16) * BV; idx += NT) {
                    const int r = b0 + 16 + idx / BV, j = idx % BV;
                    float acc = sU[r][j];
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc -= sA[r][b0 + i] * sU[b0 + i][j];
                    sU[r][j] = acc;
                }
                __syncthreads();
            }
        }

        // O = scale ((gamma*Q) S + P U): P U added on the matrix cores by the
        // waves that hold (gamma*Q) S (16-row chunks), else 4 columns per thread
        if constexpr (kMfma) {
            if (wave >= NTL && wave < 2 * NTL) {
#pragma unroll
                for (int s4 = 0; s4 < C; s4 += 4)
                    macc = __builtin_amdgcn_mfma_f32_16x16x4f32(sP[l16][s4 + lg], sU[s4 + lg][16 * mt + l16], macc, 0,
                                                                0, 0);
                if (o) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = 4 * lg + i;
                        if (m < rows) store_elem(o, ((tok0 + m) * H + h) * Dv + c0 + 16 * mt + l16, a.scale * macc[i]);
                    }
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < kRT; ++e) {
                const int idx = tid + NT * e;
                const int r = idx / (BV / 4), j = 4 * (idx % (BV / 4));
                if (idx < C * (BV / 4) && r < rows && o) {
                    f32x4 acc = qs[e];
                    for (int i = 0; i <= r; ++i) acc += sP[r][i] * *reinterpret_cast<const f32x4*>(&sU[i][j]);
                    const int64_t ob = ((tok0 + r) * H + h) * Dv + c0 + j;
#pragma unroll
                    for (int u = 0; u < 4; ++u) store_elem(o, ob + u, a.scale * acc[u]);
                }
            }
        }
        __syncthreads();

        // S <- Diag(gamma_C) S + (exp(Gamma_C - Gamma) K)^T U: 16 x 16 tiles on
        // the matrix cores for 16-row chunks (K^T as the A operand), else 4 x 4
        // tiles per thread
        if constexpr (kMfma) {
            for (int tile = wave; tile < (DK / 16) * NTL; tile += NT / 64) {
                const int tm = 16 * (tile / NTL), tn = 16 * (tile % NTL);
                f32x4 acc;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = sEd[tm + 4 * lg + i] * sS[tm + 4 * lg + i][tn + l16];
#pragma unroll
                for (int s4 = 0; s4 < C; s4 += 4)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sK[s4 + lg][tm + l16], sU[s4 + lg][tn + l16], acc, 0, 0,
                                                               0);
#pragma unroll
                for (int i = 0; i < 4; ++i) sS[tm + 4 * lg + i][tn + l16] = acc[i];
            }
        } else {
            constexpr int TJ = 4;
            for (int idx = tid; idx < (DK / 4) * (BV / TJ); idx += NT) {
                const int c = 4 * (idx / (BV / TJ)), j = TJ * (idx % (BV / TJ));
                f32x4 acc[4][TJ / 4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float d = sEd[c + u];
#pragma unroll
                    for (int w = 0; w < TJ / 4; ++w) acc[u][w] = d * *reinterpret_cast<const f32x4*>(&sS[c + u][j + 4 * w]);
                }
                for (int r = 0; r < rows; ++r) {
                    f32x4 ur[TJ / 4];
#pragma unroll
                    for (int w = 0; w < TJ / 4; ++w) ur[w] = *reinterpret_cast<const f32x4*>(&sU[r][j + 4 * w]);
                    const f32x4 kr = ld4(&sK[r][c]);
#pragma unroll
                    for (int u = 0; u < 4; ++u)
#pragma unroll
                        for (int w = 0; w < TJ / 4; ++w) acc[u][w] += kr[u] * ur[w];
                }
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int w = 0; w < TJ / 4; ++w) *reinterpret_cast<f32x4*>(&sS[c + u][j + 4 * w]) = acc[u][w];
            }
        }
        __syncthreads();
    }
    if (a.sT) {
        for (int idx = tid; idx < DK * BV; idx += NT) {
            const int r = idx / BV, c = idx % BV;
            a.sT[state_base + (int64_t)r * Dv + c0 + c] = sS[r][c];
        }
    }
}

template <int DK, int C, int BV>
hipError_t launch_bv(const ChunkArgs& a, hipStream_t s) {
    const int units = a.N * a.H;
    const dim3 grid((unsigned)(units * (a.Dv / BV)));
    if (a.bf16)
        hipLaunchKernelGGL((chunk_generic_kernel<DK, C, BV, __bf16>), grid, dim3(kGenThreads), 0, s, a);
    else
        hipLaunchKernelGGL((chunk_generic_kernel<DK, C, BV, float>), grid, dim3(kGenThreads), 0, s, a);
    return hipGetLastError();
}

// Compute units of the current device (cached per device).
int cu_count() {
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <int DK, int C, int DV>
hipError_t launch_dk_c_dv(const ChunkArgs& a, hipStream_t s) {
    constexpr int BV = gen_bv(C, DV);
    if constexpr (C == 16 && BV == 64) {
        // 32-column slices when even they leave no more workgroups than compute
        // units: twice the workgroups, each on a compute unit of its own (the
        // per-element sums are the same, so is the result)
        if ((int64_t)a.N * a.H * (a.Dv / 32) <= cu_count()) return launch_bv<DK, C, 32>(a, s);
    }
    return launch_bv<DK, C, BV>(a, s);
}

template <int DK, int C>
hipError_t launch_dk_c(const ChunkArgs& a, hipStream_t s) {
    switch (a.Dv) {
        case 16: return launch_dk_c_dv<DK, C, 16>(a, s);
        case 32: return launch_dk_c_dv<DK, C, 32>(a, s);
        default: return launch_dk_c_dv<DK, C, 64>(a, s);   // 64 and 128: slices of gen_bv(C, 64)
    }
}

template <int DK>
hipError_t launch_dk(const ChunkArgs& a, hipStream_t s) {
    switch (a.chunk) {
        case 16: return launch_dk_c<DK, 16>(a, s);
        case 32: return launch_dk_c<DK, 32>(a, s);
        case 64: return launch_dk_c<DK, 64>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_chunk_generic(const ChunkArgs& a, hipStream_t s) {
    switch (a.Dk) {
        case 16: return launch_dk<16>(a, s);
        case 32: return launch_dk<32>(a, s);
        case 64: return launch_dk<64>(a, s);
        case 128: return launch_dk<128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
