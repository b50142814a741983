// Fused chunkwise KDA forward for bf16 inputs, d_k = d_v = 128, chunk 64, on
// the gfx950 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// One workgroup (4 waves) owns one (sequence, head, BV-column slice of d_v)
// and walks the sequence chunk by chunk. The float32 state slice S
// (128 x BV) never leaves registers: wave w holds columns [w*BV/4, (w+1)*BV/4)
// as 16x16 accumulator tiles. Per chunk of 64 rows (entry state S):
//
//  phase A (state independent, all waves, through LDS)
//   Gamma  in-chunk cumulative log-decay per channel, built from 16-row
//          sub-chunks: L = Gamma - base_s inside sub-chunk s, base_s = Gamma at
//          the end of sub-chunk s-1. Since g >= -5, |L| <= 80 < ln(FLT_MAX).
//   M, P   decayed key-key / query-key products,
//            M[r][i] = beta_r sum_c k_rc k_ic e^{Gamma_rc - Gamma_ic}  (i < r)
//            P[r][i] =        sum_c q_rc k_ic e^{Gamma_rc - Gamma_ic}  (i <= r)
//          as 16x16 tiles (R >= I) of A_R . B_(R,I)^T with
//            A_R   = k_r e^{Gamma_r - base_R}  (<= 1)       (q for P)
//            B_R,I = k_i e^{base_R - Gamma_i}  (<= e^80 only when I == R)
//          so every factor stays in float range.
//   T      (I + M)^{-1}: 16x16 diagonal blocks by forward substitution, the
//          off-diagonal blocks level by level with fp32 MFMA.
//   also   gamma*K, gamma*Q, (e^{Gamma_C - Gamma} K)^T, V^T, beta, e^{Gamma_C}.
//  phase B (state dependent, each wave on its own columns, in registers)
//   Y = (gamma K) S;  X = Diag(beta)(V - Y);  U = T X
//   O = scale ((gamma Q) S + P U)
//   S <- Diag(e^{Gamma_C}) S + (e^{Gamma_C - Gamma} K)^T U
//
// This is the WY/UT-transform chunk form of the gated delta rule with a
// per-channel decay. Matrix-core operand convention: an A operand is read
// from LDS with its contraction axis permuted inside each 32-block so that
// lane group g holds logical indices {4g..4g+3, 16+4g..16+4g+3}; that is
// exactly what a pair of 16x16 float accumulator tiles holds per lane, so
// accumulators (S, X, U) feed the next product as B operands without any
// data movement. Only two facts of the instruction are relied on: A row and
// B column are lane%16, and A and B map their 8 contraction slots per lane
// group identically.
#include "device_common.hpp"
#include "launchers.hpp"

namespace kda {
namespace {

constexpr int kThreads = 256;
constexpr int kC = 64;
constexpr int kDK = 128;
constexpr int kDV = 128;

// ---- LDS map (bytes) -------------------------------------------------------
constexpr int OFF_KG = 0;                      // [64][128] bf16  gamma*K
constexpr int OFF_QH = OFF_KG + 16384;         // [64][128] bf16  gamma*Q
constexpr int OFF_KHT = OFF_QH + 16384;        // [128][64] bf16  (e^{Gc-G} K)^T
constexpr int OFF_TT = OFF_KHT + 16384;        // [64][64]  bf16  T
constexpr int OFF_PP = OFF_TT + 8192;          // [64][64]  bf16  P
constexpr int OFF_VT = OFF_PP + 8192;          // [BV][64]  bf16  V^T
template <int BV> constexpr int off_beta() { return OFF_VT + BV * 128; }       // [64] f32
template <int BV> constexpr int off_egn() { return off_beta<BV>() + 256; }     // [128] f32
template <int BV> constexpr int off_sub() { return off_egn<BV>() + 512; }      // [4][128] f32
template <int BV> constexpr int off_scr() { return off_sub<BV>() + 2048; }     // scratch union
// scratch, phase A products: KA | QA | BT[10]
constexpr int SCR_KA = 0;
constexpr int SCR_QA = 16384;
constexpr int SCR_BT = 32768;                  // 10 tiles [16][128] bf16, 4096 B each
constexpr int SCR_SIZE = SCR_BT + 10 * 4096;   // 73728
// scratch, inverse: MF | TF, float [64][FST]
constexpr int FST = 68;
constexpr int SCR_MF = 0;
constexpr int SCR_TF = 64 * FST * 4;
// scratch also holds the output staging [64][BV] bf16 and, before the chunk
// loop, the packed sequence lengths (<= 256 ints)
template <int BV> constexpr int lds_bytes() { return off_scr<BV>() + SCR_SIZE; }
static_assert(lds_bytes<128>() <= 163840, "LDS budget");
static_assert(2 * 64 * FST * 4 <= SCR_SIZE, "inverse scratch");

// B tile (R, I), I <= R, of the decayed-product operands
__host__ __device__ constexpr int bt(int R, int I) { return R * (R + 1) / 2 + I; }

__device__ __forceinline__ int perm32(int x) {  // position of logical index x inside its 32-block
    return ((x & 15) >> 2) * 8 + (x >> 4) * 4 + (x & 3);
}
__device__ __forceinline__ int phys_col(int c) { return (c & ~31) + perm32(c & 31); }
// [rows][128] bf16: 16 chunks of 16 B per row, chunk index XOR (row % 16)
__device__ __forceinline__ int a256(int row, int chunk) { return row * 256 + ((chunk ^ (row & 15)) << 4); }
// [rows][64] bf16: 8 chunks of 16 B per row, chunk index XOR (row % 8)
__device__ __forceinline__ int a128(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }
// V^T [BV][64] bf16: 16 pieces of 8 B per row, piece index XOR (row % 16)
__device__ __forceinline__ int vt_off(int row, int piece) { return row * 128 + ((piece ^ (row & 15)) << 3); }
__device__ __forceinline__ int a128_elem(int row, int col) {
    const int p = phys_col(col);
    return a128(row, p >> 3) + ((p & 7) << 1);
}

__device__ __forceinline__ bf16x8 lds_frag(const char* smem, int off) {
    return *reinterpret_cast<const bf16x8*>(smem + off);
}
__device__ __forceinline__ bf16x8 pack_frag(const f32x4& lo, const f32x4& hi) {
    bf16x8 r;
    r[0] = (__bf16)lo[0]; r[1] = (__bf16)lo[1]; r[2] = (__bf16)lo[2]; r[3] = (__bf16)lo[3];
    r[4] = (__bf16)hi[0]; r[5] = (__bf16)hi[1]; r[6] = (__bf16)hi[2]; r[7] = (__bf16)hi[3];
    return r;
}
__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void st_bf16(char* smem, int off, float v) {
    *reinterpret_cast<uint16_t*>(smem + off) = f32_to_bf16_bits(v);
}
__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d) {
    return make_uint2(pack2_bf16(a, b), pack2_bf16(c, d));
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Map block index -> work item so that the BV-slices of one (sequence, head)
// land on the same XCD (blocks are dealt round-robin over the 8 XCDs) and
// are dispatched together: they read the same q, k, g, which that XCD's L2
// can then serve once.
__device__ __forceinline__ int remap_block(int b, int units, int nvt) {
    const int per = 8 * nvt;
    const int full = (units / 8) * per;
    if (b >= full) return b;
    const int grp = b / per, rem = b % per;
    return (grp * 8 + (rem & 7)) * nvt + (rem >> 3);
}

struct ChunkRegs {
    uint4 q[4], k[4], g[4], v[4];
    float beta;
};

// Global -> register loads of one chunk (rows >= `rows` read as zero).
// Thread layout: wave w = sub-chunk w; lane (cg = lane%16, j4 = lane/16)
// holds rows 16w+4*j4+[0..3], channels 8*cg..8*cg+7 (16-byte loads; each
// row's 256 bytes are read by 16 consecutive lanes).
template <int BV>
__device__ __forceinline__ void load_chunk(ChunkRegs& R, const ChunkArgs& a, int64_t tok0, int rows,
                                           int h, int vt, int tid) {
    const int w = tid >> 6, lane = tid & 63, cg = lane & 15, j4 = lane >> 4;
    const uint16_t* q = static_cast<const uint16_t*>(a.q);
    const uint16_t* k = static_cast<const uint16_t*>(a.k);
    const uint16_t* g = static_cast<const uint16_t*>(a.g);
    const uint16_t* v = static_cast<const uint16_t*>(a.v);
    const uint16_t* beta = static_cast<const uint16_t*>(a.beta);
    const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + 4 * j4 + i;
        if (r < rows) {
            const int64_t e = ((tok0 + r) * a.H + h) * kDK + 8 * cg;
            R.q[i] = *reinterpret_cast<const uint4*>(q + e);
            R.k[i] = *reinterpret_cast<const uint4*>(k + e);
            R.g[i] = *reinterpret_cast<const uint4*>(g + e);
        } else {
            R.q[i] = z;
            R.k[i] = z;
            R.g[i] = z;
        }
    }
    constexpr int CB = BV / 8;  // 16-byte column blocks per row of the V slice
    if (tid < 16 * CB) {
        const int rq = tid / CB, cb = tid % CB;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * rq + i;
            R.v[i] = (r < rows) ? *reinterpret_cast<const uint4*>(
                                      v + ((tok0 + r) * a.H + h) * kDV + vt * BV + 8 * cb)
                                : z;
        }
    }
    if (tid < kC) R.beta = (tid < rows) ? bf16_bits_to_f32(beta[(tok0 + tid) * a.H + h]) : 0.f;
}

template <int BV>
__global__ __launch_bounds__(kThreads, 1) void chunk_mfma_kernel(ChunkArgs a) {
    constexpr int NVT = kDV / BV;
    constexpr int NW = BV / 4;       // state columns per wave
    constexpr int NCT = NW / 16;     // 16-column tiles per wave
    constexpr int CB = BV / 8;
    constexpr int OFF_BETA = off_beta<BV>();
    constexpr int OFF_EGN = off_egn<BV>();
    constexpr int OFF_SUB = off_sub<BV>();
    constexpr int OFF_SCR = off_scr<BV>();
    __shared__ __attribute__((aligned(16))) char smem[lds_bytes<BV>()];
    char* scr = smem + OFF_SCR;
    float* sBeta = reinterpret_cast<float*>(smem + OFF_BETA);
    float* sEgn = reinterpret_cast<float*>(smem + OFF_EGN);
    float* sSub = reinterpret_cast<float*>(smem + OFF_SUB);
    float* sMF = reinterpret_cast<float*>(scr + SCR_MF);
    float* sTF = reinterpret_cast<float*>(scr + SCR_TF);

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, li = lane & 15, lg = lane >> 4;
    const int units = a.N * a.H;

    // ---- work item ----------------------------------------------------------
    const int wi = remap_block(blockIdx.x, units, NVT);
    const int unit = wi / NVT, vt = wi % NVT;
    int n = unit / a.H;
    const int h = unit % a.H;
    if (a.cu && a.N <= 256) {
        // packed batch: the rank-n longest sequence (ties by index) goes first
        int* lens = reinterpret_cast<int*>(scr);
        int* pick = reinterpret_cast<int*>(smem + OFF_SUB);
        if (tid < a.N) lens[tid] = a.cu[tid + 1] - a.cu[tid];
        __syncthreads();
        if (tid < a.N) {
            const int my = lens[tid];
            int rank = 0;
            for (int s = 0; s < a.N; ++s) {
                const int ls = lens[s];
                rank += (ls > my) || (ls == my && s < tid);
            }
            if (rank == n) *pick = tid;
        }
        __syncthreads();
        n = *pick;
        __syncthreads();
    }
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
    const int nchunks = (int)((len + kC - 1) / kC);
    const int64_t state_base = ((int64_t)n * a.H + h) * kDK * kDV;
    const int cw = w * NW;                 // first slice column of this wave
    const int col0 = vt * BV + cw;         // first d_v column of this wave

    // upper blocks of T and P are never written and must read as zero
    for (int i = tid; i < 2 * 8192 / 16; i += kThreads)
        reinterpret_cast<uint4*>(smem + OFF_TT)[i] = make_uint4(0, 0, 0, 0);

    // ---- state tiles in registers -------------------------------------------
    f32x4 S[8][NCT];
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                S[rt][ct][j] = a.s0 ? a.s0[state_base + (int64_t)(16 * rt + 4 * lg + j) * kDV + col0 + 16 * ct + li]
                                    : 0.f;

    ChunkRegs R;
    if (nchunks > 0) load_chunk<BV>(R, a, b * (int64_t)a.T + bos, (int)(len < kC ? len : kC), h, vt, tid);

    const int cg = li;       // phase A: channel group (8 channels)
    const int j4 = lg;       // phase A: row quad inside the sub-chunk
    for (int ci = 0; ci < nchunks; ++ci) {
        const int64_t tok0 = b * (int64_t)a.T + bos + (int64_t)ci * kC;
        const int64_t left = len - (int64_t)ci * kC;
        const int rows = (int)(left < kC ? left : kC);

        // ================= A1: cumulative log-decay ==========================
        float L[4][8];
        {
            float gf[4][8];
#pragma unroll
            for (int i = 0; i < 4; ++i) unpack8(R.g[i], gf[i]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float pre[4];
                pre[0] = gf[0][e];
#pragma unroll
                for (int i = 1; i < 4; ++i) pre[i] = pre[i - 1] + gf[i][e];
                const float tot = pre[3];
                float acc = tot;
                float y = __shfl_up(acc, 16);
                if (j4 >= 1) acc += y;
                y = __shfl_up(acc, 32);
                if (j4 >= 2) acc += y;
                const float excl = acc - tot;
#pragma unroll
                for (int i = 0; i < 4; ++i) L[i][e] = excl + pre[i];
                if (j4 == 3) sSub[w * 128 + 8 * cg + e] = acc;   // sub-chunk total
            }
        }
        __syncthreads();   // (1) sub-chunk totals visible; output staging of the last chunk consumed

        // per-channel factors for this thread's 8 channels
        float e_base[8], e_tot[8], e_hat[8], e_b2[8], e_b3[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float t0 = sSub[0 * 128 + 8 * cg + e], t1 = sSub[1 * 128 + 8 * cg + e];
            const float t2 = sSub[2 * 128 + 8 * cg + e], t3 = sSub[3 * 128 + 8 * cg + e];
            const float base1 = t0, base2 = t0 + t1, base3 = t0 + t1 + t2, gn = base3 + t3;
            const float tw = (w == 0) ? t0 : (w == 1) ? t1 : (w == 2) ? t2 : t3;
            const float bw = (w == 0) ? 0.f : (w == 1) ? base1 : (w == 2) ? base2 : base3;
            const float bw1 = bw + tw;                            // base_{w+1}
            e_base[e] = fast_exp(bw);                             // e^{base_w}
            e_tot[e] = fast_exp(tw);                              // e^{tot_w}
            e_hat[e] = fast_exp(gn - bw1);                        // e^{Gamma_C - base_{w+1}}
            e_b2[e] = fast_exp(((w == 0) ? base2 : base3) - bw1); // e^{base_{w+2} - base_{w+1}}
            e_b3[e] = fast_exp(base3 - bw1);                      // e^{base_3 - base_1} (w == 0)
            if (w == 0 && j4 == 0) sEgn[8 * cg + e] = fast_exp(gn);
        }

        // ================= A2: elementwise operands -> LDS ===================
        {
            const int x0 = 8 * (cg & 3), x1 = x0 + 4;
            const int p0 = 32 * (cg >> 2) + ((x0 & 15) >> 2) * 8 + (x0 >> 4) * 4;
            const int p1 = 32 * (cg >> 2) + ((x1 & 15) >> 2) * 8 + (x1 >> 4) * 4;
            auto put256 = [&](char* base, int row, const float* f) {
                *reinterpret_cast<uint2*>(base + a256(row, p0 >> 3) + ((p0 & 7) << 1)) =
                    pack4_bf16(f[0], f[1], f[2], f[3]);
                *reinterpret_cast<uint2*>(base + a256(row, p1 >> 3) + ((p1 & 7) << 1)) =
                    pack4_bf16(f[4], f[5], f[6], f[7]);
            };
            float kh[4][8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * w + 4 * j4 + i;                // chunk row
                const int tr = 4 * j4 + i;                        // row inside a 16-row tile
                float kf[8], qf[8];
                unpack8(R.k[i], kf);
                unpack8(R.q[i], qf);
                float ka[8], qa[8], kg[8], qh[8], kb[8], kc[8], t2[8], t3[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float eL = fast_exp(L[i][e]);
                    const float eNL = fast_exp(-L[i][e]);
                    ka[e] = kf[e] * eL;
                    qa[e] = qf[e] * eL;
                    kg[e] = ka[e] * e_base[e];
                    qh[e] = qa[e] * e_base[e];
                    kb[e] = kf[e] * eNL;
                    kc[e] = kb[e] * e_tot[e];                     // k e^{base_{w+1} - Gamma}
                    kh[i][e] = kc[e] * e_hat[e];                  // k e^{Gamma_C - Gamma}
                    t2[e] = kc[e] * e_b2[e];
                    t3[e] = kc[e] * e_b3[e];
                }
                put256(scr + SCR_KA, r, ka);
                put256(scr + SCR_QA, r, qa);
                put256(smem + OFF_KG, r, kg);
                put256(smem + OFF_QH, r, qh);
                put256(scr + SCR_BT + bt(w, w) * 4096, tr, kb);
                if (w <= 2) put256(scr + SCR_BT + bt(w + 1, w) * 4096, tr, kc);
                if (w <= 1) put256(scr + SCR_BT + bt(w + 2, w) * 4096, tr, t2);
                if (w == 0) put256(scr + SCR_BT + bt(3, 0) * 4096, tr, t3);
            }
            // (e^{Gamma_C - Gamma} K)^T: for channel c, the 4 rows of this thread
            // are 4 consecutive positions of row c
            const int rr = 16 * w + 4 * j4;                       // first chunk row
            const int pr = 32 * (rr >> 5) + perm32(rr & 31);      // its physical position
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int c = 8 * cg + e;
                *reinterpret_cast<uint2*>(smem + OFF_KHT + a128(c, pr >> 3) + ((pr & 7) << 1)) =
                    pack4_bf16(kh[0][e], kh[1][e], kh[2][e], kh[3][e]);
            }
            // V^T and beta
            if (tid < 16 * CB) {
                const int rq = tid / CB, cb = tid % CB;
                float vf[4][8];
#pragma unroll
                for (int i = 0; i < 4; ++i) unpack8(R.v[i], vf[i]);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int row = 8 * cb + e;
                    *reinterpret_cast<uint2*>(smem + OFF_VT + vt_off(row, rq)) =
                        pack4_bf16(vf[0][e], vf[1][e], vf[2][e], vf[3][e]);
                }
            }
            if (tid < kC) sBeta[tid] = R.beta;
        }
        __syncthreads();   // (2) phase-A operands visible

        // prefetch the next chunk into registers; consumed one iteration later
        if (ci + 1 < nchunks) {
            const int64_t left1 = left - kC;
            load_chunk<BV>(R, a, tok0 + kC, (int)(left1 < kC ? left1 : kC), h, vt, tid);
        }

        // ================= A3: M and P tiles ==================================
        // wave w: M row block w (tiles I <= w) and P row block 3-w (tiles I <= 3-w)
        f32x4 macc[4], pacc[4];
        {
            bf16x8 af[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) af[kk] = lds_frag(scr + SCR_KA, a256(16 * w + li, 4 * kk + lg));
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                macc[I] = zero4();
                if (I <= w) {
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        macc[I] = mfma_bf16(af[kk], lds_frag(scr + SCR_BT + bt(w, I) * 4096, a256(li, 4 * kk + lg)),
                                            macc[I]);
                }
            }
            const int RP = 3 - w;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) af[kk] = lds_frag(scr + SCR_QA, a256(16 * RP + li, 4 * kk + lg));
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                pacc[I] = zero4();
                if (I <= RP) {
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        pacc[I] = mfma_bf16(af[kk], lds_frag(scr + SCR_BT + bt(RP, I) * 4096, a256(li, 4 * kk + lg)),
                                            pacc[I]);
                }
            }
        }
        __syncthreads();   // (3) operand scratch fully read; MF/TF may overwrite it

        {
            const int RP = 3 - w;
#pragma unroll
            for (int I = 0; I < 4; ++I) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (I <= w) {
                        const int r = 16 * w + 4 * lg + j, i = 16 * I + li;
                        sMF[r * FST + i] = (i < r) ? sBeta[r] * macc[I][j] : 0.f;
                    }
                    if (I <= RP) {
                        const int r = 16 * RP + 4 * lg + j, i = 16 * I + li;
                        st_bf16(smem + OFF_PP, a128_elem(r, i), (i <= r) ? pacc[I][j] : 0.f);
                    }
                }
            }
        }
        __syncthreads();   // (4) M visible

        // ================= A4: T = (I + M)^{-1} ================================
        {
            // diagonal block w: lane column li, forward substitution down the rows
            float t[16];
            const float* mrow = sMF + (16 * w) * FST + 16 * w;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == li) ? 1.f : 0.f;
#pragma unroll
                for (int i = 0; i < r; ++i) acc = fmaf(-mrow[r * FST + i], t[i], acc);
                t[r] = acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if ((r >> 2) == lg) {
                    sTF[(16 * w + r) * FST + 16 * w + li] = t[r];
                    st_bf16(smem + OFF_TT, a128_elem(16 * w + r, 16 * w + li), t[r]);
                }
            }
        }
#pragma unroll
        for (int d = 1; d < 4; ++d) {
            __syncthreads();   // (5,6,7) blocks of the previous level visible
            if (w < 4 - d) {
                const int Rb = w + d, Ib = w;
                f32x4 z = zero4();
                for (int J = Ib; J < Rb; ++J) {
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        z = mfma_f32(sMF[(16 * Rb + li) * FST + 16 * J + 4 * lg + s],
                                     sTF[(16 * J + 4 * lg + s) * FST + 16 * Ib + li], z);
                }
                f32x4 tr = zero4();
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    tr = mfma_f32(sTF[(16 * Rb + li) * FST + 16 * Rb + 4 * lg + s], z[s], tr);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 16 * Rb + 4 * lg + j, i = 16 * Ib + li;
                    sTF[r * FST + i] = -tr[j];
                    st_bf16(smem + OFF_TT, a128_elem(r, i), -tr[j]);
                }
            }
        }
        __syncthreads();   // (8) T complete

        // ================= B: state-dependent chain, per wave ==================
        {
            bf16x8 sb[4][NCT];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) sb[kk][ct] = pack_frag(S[2 * kk][ct], S[2 * kk + 1][ct]);

            f32x4 y[4][NCT], qs[4][NCT];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    y[rt][ct] = zero4();
                    qs[rt][ct] = zero4();
                }
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const bf16x8 ak = lds_frag(smem + OFF_KG, a256(16 * rt + li, 4 * kk + lg));
                    const bf16x8 aq = lds_frag(smem + OFF_QH, a256(16 * rt + li, 4 * kk + lg));
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        y[rt][ct] = mfma_bf16(ak, sb[kk][ct], y[rt][ct]);
                        qs[rt][ct] = mfma_bf16(aq, sb[kk][ct], qs[rt][ct]);
                    }
                }
            }
            // X = Diag(beta) (V - Y), reusing y
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const f32x4 bb = *reinterpret_cast<const f32x4*>(sBeta + 16 * rt + 4 * lg);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    const uint2 vv = *reinterpret_cast<const uint2*>(smem + OFF_VT + vt_off(cw + 16 * ct + li, 4 * rt + lg));
                    y[rt][ct][0] = bb[0] * (__uint_as_float(vv.x << 16) - y[rt][ct][0]);
                    y[rt][ct][1] = bb[1] * (__uint_as_float(vv.x & 0xffff0000u) - y[rt][ct][1]);
                    y[rt][ct][2] = bb[2] * (__uint_as_float(vv.y << 16) - y[rt][ct][2]);
                    y[rt][ct][3] = bb[3] * (__uint_as_float(vv.y & 0xffff0000u) - y[rt][ct][3]);
                }
            }
            bf16x8 xb[2][NCT];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) xb[kk][ct] = pack_frag(y[2 * kk][ct], y[2 * kk + 1][ct]);
            // U = T X (T lower triangular: row block rt needs contraction blocks <= rt)
            f32x4 u[4][NCT];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) u[rt][ct] = zero4();
#pragma unroll
                for (int kk = 0; kk <= (rt >> 1); ++kk) {
                    const bf16x8 at = lds_frag(smem + OFF_TT, a128(16 * rt + li, 4 * kk + lg));
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) u[rt][ct] = mfma_bf16(at, xb[kk][ct], u[rt][ct]);
                }
            }
            bf16x8 ub[2][NCT];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) ub[kk][ct] = pack_frag(u[2 * kk][ct], u[2 * kk + 1][ct]);
            // O = scale ((gamma Q) S + P U) -> output staging
            char* ost = scr;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
                for (int kk = 0; kk <= (rt >> 1); ++kk) {
                    const bf16x8 ap = lds_frag(smem + OFF_PP, a128(16 * rt + li, 4 * kk + lg));
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) qs[rt][ct] = mfma_bf16(ap, ub[kk][ct], qs[rt][ct]);
                }
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        st_bf16(ost, ((16 * rt + 4 * lg + j) * BV + cw + 16 * ct + li) * 2, a.scale * qs[rt][ct][j]);
            }
            // S <- Diag(e^{Gamma_C}) S + (e^{Gamma_C - Gamma} K)^T U
#pragma unroll
            for (int rt = 0; rt < 8; ++rt) {
                const f32x4 eg = *reinterpret_cast<const f32x4*>(sEgn + 16 * rt + 4 * lg);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) S[rt][ct] *= eg;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const bf16x8 ah = lds_frag(smem + OFF_KHT, a128(16 * rt + li, 4 * kk + lg));
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) S[rt][ct] = mfma_bf16(ah, ub[kk][ct], S[rt][ct]);
                }
            }
        }
        __syncthreads();   // (9) output staging complete

        // ---- coalesced output store (rows past the sequence end are skipped) ---
        {
            uint16_t* o = static_cast<uint16_t*>(a.o);
            for (int it = tid; it < kC * CB; it += kThreads) {
                const int r = it / CB, cb = it % CB;
                if (r < rows) {
                    const uint4 val = *reinterpret_cast<const uint4*>(scr + (r * BV + 8 * cb) * 2);
                    *reinterpret_cast<uint4*>(o + ((tok0 + r) * a.H + h) * kDV + vt * BV + 8 * cb) = val;
                }
            }
        }
    }

    if (a.sT) {
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    a.sT[state_base + (int64_t)(16 * rt + 4 * lg + j) * kDV + col0 + 16 * ct + li] = S[rt][ct][j];
    }
}

}  // namespace

bool chunk_mfma_supported(const ChunkArgs& a) {
    return a.bf16 && a.Dk == kDK && a.Dv == kDV && a.chunk == kC;
}

// Column-slice width: BV = 64 doubles the workgroup count (two slices per
// head), which pays while (sequences x heads) leaves most of the 256 CUs idle.
hipError_t launch_chunk_mfma(const ChunkArgs& a, hipStream_t s) {
    const int units = a.N * a.H;
    if (units <= 256) {
        hipLaunchKernelGGL(chunk_mfma_kernel<64>, dim3((unsigned)(units * 2)), dim3(kThreads), 0, s, a);
    } else {
        hipLaunchKernelGGL(chunk_mfma_kernel<128>, dim3((unsigned)units), dim3(kThreads), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace kda
