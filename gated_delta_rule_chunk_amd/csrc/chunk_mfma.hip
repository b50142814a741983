// Fused chunkwise KDA forward for bf16 inputs, d_k = d_v = 128, chunk 64, on
// the gfx950 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// One workgroup (4 waves) owns one (sequence, head, BV-column slice of d_v)
// and walks the sequence chunk by chunk. The float32 state slice S
// (128 x BV) never leaves registers: wave w holds columns [w*BV/4, (w+1)*BV/4)
// as 16x16 accumulator tiles. Per chunk of 64 rows (entry state S):
//
//  phase A (state independent, all waves, through LDS)
//   Gamma  in-chunk cumulative log-decay per channel (kept in log2 units),
//          built from 16-row sub-chunks: L = Gamma - base_s inside sub-chunk
//          s, base_s = Gamma at the end of sub-chunk s-1, tot_s = its sum.
//          Since g >= -5, |L| <= 80 < ln(FLT_MAX); every per-channel factor
//          (e^{base_s}, e^{Gamma_C - base_{s+1}}, ...) is a product of the four
//          values e^{tot_s} <= 1, so it only ever underflows towards a value
//          that is itself below float range.
//   M, P   decayed key-key / query-key products,
//            M[r][i] = beta_r sum_c k_rc k_ic e^{Gamma_rc - Gamma_ic}  (i < r)
//            P[r][i] =        sum_c q_rc k_ic e^{Gamma_rc - Gamma_ic}  (i <= r)
//          as 16x16 tiles (R >= I) of A_R . B_(R,I)^T with
//            A_R   = k_r e^{Gamma_r - base_R}  (<= 1)       (q for P)
//            B_R,I = k_i e^{base_R - Gamma_i}  (<= e^80 only when I == R)
//   T      (I + M)^{-1}: 16x16 diagonal blocks by forward substitution, the
//          off-diagonal blocks level by level with fp32 MFMA.
//   also   gamma*K, gamma*Q, (e^{Gamma_C - Gamma} K)^T, V^T, beta, e^{Gamma_C}.
//  phase B (state dependent, each wave on its own columns, in registers)
//   Y = (gamma K) S;  X = Diag(beta)(V - Y);  U = T X
//   O = scale ((gamma Q) S + P U), computed transposed so that each lane
//       holds 4 consecutive output columns and stores them straight to HBM
//   S <- Diag(e^{Gamma_C}) S + (e^{Gamma_C - Gamma} K)^T U
//
// This is the WY/UT-transform chunk form of the gated delta rule with a
// per-channel decay. Matrix-core operand convention: an operand read from
// LDS has its contraction axis permuted inside each 32-block so that lane
// group g holds logical indices {4g..4g+3, 16+4g..16+4g+3}; that is exactly
// what a pair of 16x16 float accumulator tiles holds per lane, so
// accumulators (S, X, U) feed the next product as A or B operands without
// any data movement. Only two facts of the instruction are relied on: A row
// and B column are lane%16, and A and B map their 8 contraction slots per
// lane group identically. Swapping the A and B operands of a product yields
// its transpose, which is how row-contiguous outputs are produced.
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
// scratch also stages the initial / final state slice ([128][BV] f32) and,
// before the chunk loop, the packed sequence lengths (<= 256 ints)
template <int BV> constexpr int lds_bytes() { return off_scr<BV>() + SCR_SIZE; }
static_assert(lds_bytes<128>() <= 163840, "LDS budget");
static_assert(2 * 64 * FST * 4 <= SCR_SIZE, "inverse scratch");
static_assert(128 * 128 * 4 <= SCR_SIZE, "state staging");

// B tile (R, I), I <= R, of the decayed-product operands
__host__ __device__ constexpr int bt(int R, int I) { return R * (R + 1) / 2 + I; }

__device__ __forceinline__ int perm32(int x) {  // position of logical index x inside its 32-block
    return ((x & 15) >> 2) * 8 + (x >> 4) * 4 + (x & 3);
}
// [rows][128] bf16: 16 chunks of 16 B per row, chunk index XOR (row % 16)
__device__ __forceinline__ int a256(int row, int chunk) { return row * 256 + ((chunk ^ (row & 15)) << 4); }
// [rows][64] bf16: 8 chunks of 16 B per row, chunk index XOR (row % 8)
__device__ __forceinline__ int a128(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }
// (e^{Gc-G} K)^T [128][64] bf16: chunk index XOR ((row ^ row/8) % 8), which
// spreads both its transposed writes (rows 8 apart) and its fragment reads
__device__ __forceinline__ int kht_off(int row, int chunk) {
    return row * 128 + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}
// V^T [BV][64] bf16: 16 pieces of 8 B per row, piece index XOR (row % 16)
__device__ __forceinline__ int vt_off(int row, int piece) { return row * 128 + ((piece ^ (row & 15)) << 3); }

__device__ __forceinline__ bf16x8 lds_frag(const char* smem, int off) {
    return *reinterpret_cast<const bf16x8*>(smem + off);
}
__device__ __forceinline__ bf16x8 pack_frag(const f32x4& lo, const f32x4& hi) {
    const bf16x8 r = {(__bf16)lo[0], (__bf16)lo[1], (__bf16)lo[2], (__bf16)lo[3],
                      (__bf16)hi[0], (__bf16)hi[1], (__bf16)hi[2], (__bf16)hi[3]};
    return r;
}
__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d) {
    return make_uint2(pack2_bf16(a, b), pack2_bf16(c, d));
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

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
    uint32_t beta;   // raw bf16 bits
};

// Global -> register loads of one chunk. Every load is unconditional: rows at
// or past `rows` re-read row rows-1 (always a valid address) and are zeroed
// where the registers are consumed, so no load sits behind a branch or a
// pointer select and none has to complete before the next chunk's work.
// Thread layout: wave w = sub-chunk w; lane (cg = lane%16, j4 = lane/16)
// holds rows 16w+4*j4+[0..3], channels 8*cg..8*cg+7 (16-byte loads; each
// row's 256 bytes are read by 16 consecutive lanes).
template <int BV>
__device__ __forceinline__ void load_chunk(ChunkRegs& R, const ChunkArgs& a, int64_t tok0, int rows,
                                           int h, int vt, int w, int tid) {
    const int lane = tid & 63, cg = lane & 15, j4 = lane >> 4;
    const uint16_t* q = static_cast<const uint16_t*>(a.q);
    const uint16_t* k = static_cast<const uint16_t*>(a.k);
    const uint16_t* g = static_cast<const uint16_t*>(a.g);
    const uint16_t* v = static_cast<const uint16_t*>(a.v);
    const uint16_t* beta = static_cast<const uint16_t*>(a.beta);
    const int last = rows - 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = min(16 * w + 4 * j4 + i, last);
        const int64_t e = ((tok0 + r) * a.H + h) * kDK + 8 * cg;
        R.q[i] = *reinterpret_cast<const uint4*>(q + e);
        R.k[i] = *reinterpret_cast<const uint4*>(k + e);
        R.g[i] = *reinterpret_cast<const uint4*>(g + e);
    }
    constexpr int CB = BV / 8;  // 16-byte column blocks per row of the V slice
    const int vi = tid % (16 * CB);
    const int rq = vi / CB, cb = vi % CB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = min(4 * rq + i, last);
        R.v[i] = *reinterpret_cast<const uint4*>(v + ((tok0 + r) * a.H + h) * kDV + vt * BV + 8 * cb);
    }
    R.beta = beta[(tok0 + min(lane, last)) * a.H + h];
}

__device__ __forceinline__ uint4 keep_if(bool ok, const uint4& u) {
    return ok ? u : make_uint4(0, 0, 0, 0);
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
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
    const int lane = tid & 63, li = lane & 15, lg = lane >> 4;
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

    // upper blocks of T and P are never written and must read as zero
    for (int i = tid; i < 2 * 8192 / 16; i += kThreads)
        reinterpret_cast<uint4*>(smem + OFF_TT)[i] = make_uint4(0, 0, 0, 0);

    // ---- state tiles in registers -------------------------------------------
    // The state slice (128 x BV fp32) moves between HBM and registers through
    // LDS so that the global accesses are coalesced 16-byte rows along d_v.
    f32x4 S[8][NCT];
    if (a.s0) {
        float* stage = reinterpret_cast<float*>(scr);          // [128][BV] f32
        __syncthreads();
        for (int it = tid; it < kDK * BV / 4; it += kThreads) {
            const int r = it / (BV / 4), c4 = it % (BV / 4);
            *reinterpret_cast<f32x4*>(stage + r * BV + 4 * c4) =
                *reinterpret_cast<const f32x4*>(a.s0 + state_base + (int64_t)r * kDV + vt * BV + 4 * c4);
        }
        __syncthreads();
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int j = 0; j < 4; ++j) S[rt][ct][j] = stage[(16 * rt + 4 * lg + j) * BV + cw + 16 * ct + li];
    } else {
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) S[rt][ct] = zero4();
    }

    // ---- per-thread LDS offsets, fixed for the whole loop --------------------
    const int cg = li;       // phase A: channel group (8 channels)
    const int j4 = lg;       // phase A: row quad inside the sub-chunk
    // phase A row-major writes: rows 4*j4+i of a 16-row block, two 8-byte halves
    int offw[4][2];
    {
        const int x0 = 8 * (cg & 3), x1 = x0 + 4;
        const int p0 = 32 * (cg >> 2) + ((x0 & 15) >> 2) * 8 + (x0 >> 4) * 4;
        const int p1 = 32 * (cg >> 2) + ((x1 & 15) >> 2) * 8 + (x1 >> 4) * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tr = 4 * j4 + i;
            offw[i][0] = a256(tr, p0 >> 3) + ((p0 & 7) << 1);
            offw[i][1] = a256(tr, p1 >> 3) + ((p1 & 7) << 1);
        }
    }
    int offkht[8];   // (e^{Gc-G} K)^T: row = channel 8cg+e, 4 chunk rows 16w+4j4..+3
    {
        const int rr = 16 * w + 4 * j4;
        const int pr = 32 * (rr >> 5) + perm32(rr & 31);
#pragma unroll
        for (int e = 0; e < 8; ++e) offkht[e] = kht_off(8 * cg + e, pr >> 3) + ((pr & 7) << 1);
    }
    // phase B fragment reads (the row-block offset is added as a constant)
    int offA256[4], offA128[2], offKH[2][4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) offA256[kk] = li * 256 + (((4 * kk + lg) ^ li) << 4);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        offA128[kk] = li * 128 + (((4 * kk + lg) ^ (li & 7)) << 4);
#pragma unroll
        for (int v2 = 0; v2 < 4; ++v2)   // row 16rt+li has swizzle (li ^ li/8 ^ 2rt) % 8
            offKH[kk][v2] = li * 128 + (((4 * kk + lg) ^ (((li & 7) ^ (li >> 3) ^ (2 * v2)) & 7)) << 4);
    }

    ChunkRegs R;
    if (nchunks > 0) load_chunk<BV>(R, a, b * (int64_t)a.T + bos, (int)(len < kC ? len : kC), h, vt, w, tid);

    for (int ci = 0; ci < nchunks; ++ci) {
        const int64_t tok0 = b * (int64_t)a.T + bos + (int64_t)ci * kC;
        const int64_t left = len - (int64_t)ci * kC;
        const int rows = (int)(left < kC ? left : kC);

        // ================= A1: cumulative log2-decay ==========================
        float L[4][8];
        {
            float gf[4][8];
#pragma unroll
            for (int i = 0; i < 4; ++i) unpack8(keep_if(16 * w + 4 * j4 + i < rows, R.g[i]), gf[i]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float pre[4];
                pre[0] = gf[0][e] * kLog2e;
#pragma unroll
                for (int i = 1; i < 4; ++i) pre[i] = fmaf(gf[i][e], kLog2e, pre[i - 1]);
                const float tot = pre[3];
                float acc = tot;
                float y = __shfl_up(acc, 16);
                if (j4 >= 1) acc += y;
                y = __shfl_up(acc, 32);
                if (j4 >= 2) acc += y;
                const float excl = acc - tot;
#pragma unroll
                for (int i = 0; i < 4; ++i) L[i][e] = excl + pre[i];
                if (j4 == 3) sSub[w * 128 + 8 * cg + e] = exp2_fast(acc);   // e^{tot_w}
            }
        }
        __syncthreads();   // (1) sub-chunk factors visible; the previous phase B is done

        // per-channel factors for this thread's 8 channels, all products of e^{tot_s}
        float f_base[8], f_tot[8], f_hat[8], f_b2[8], f_b3[8];
        {
            f32x4 et[4][2];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                et[s][0] = *reinterpret_cast<const f32x4*>(sSub + s * 128 + 8 * cg);
                et[s][1] = *reinterpret_cast<const f32x4*>(sSub + s * 128 + 8 * cg + 4);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float t0 = et[0][e >> 2][e & 3], t1 = et[1][e >> 2][e & 3];
                const float t2 = et[2][e >> 2][e & 3], t3 = et[3][e >> 2][e & 3];
                float fb, ft, fh, f2, f3;
                if (w == 0) {
                    fb = 1.f; ft = t0; fh = t1 * t2 * t3; f2 = t1; f3 = t1 * t2;
                } else if (w == 1) {
                    fb = t0; ft = t1; fh = t2 * t3; f2 = t2; f3 = 0.f;
                } else if (w == 2) {
                    fb = t0 * t1; ft = t2; fh = t3; f2 = 0.f; f3 = 0.f;
                } else {
                    fb = t0 * t1 * t2; ft = t3; fh = 1.f; f2 = 0.f; f3 = 0.f;
                }
                f_base[e] = fb;     // e^{base_w}
                f_tot[e] = ft;      // e^{tot_w}
                f_hat[e] = fh;      // e^{Gamma_C - base_{w+1}}
                f_b2[e] = f2;       // e^{base_{w+2} - base_{w+1}}
                f_b3[e] = f3;       // e^{base_3 - base_1}
                if (w == 0 && j4 == 0) sEgn[8 * cg + e] = t0 * t1 * t2 * t3;   // e^{Gamma_C}
            }
        }

        // ================= A2: elementwise operands -> LDS ===================
        {
            char* const rowblk = smem + 16 * w * 256;          // row block w of KG / QH
            char* const kablk = scr + 16 * w * 256;
            float kh[4][8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = 16 * w + 4 * j4 + i < rows;
                float kf[8], qf[8];
                unpack8(keep_if(ok, R.k[i]), kf);
                unpack8(keep_if(ok, R.q[i]), qf);
                float ka[8], qa[8], kg[8], qh[8], kb[8], kc[8], t2[8], t3[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float eL = exp2_fast(L[i][e]);
                    const float eNL = exp2_fast(-L[i][e]);
                    ka[e] = kf[e] * eL;
                    qa[e] = qf[e] * eL;
                    kg[e] = ka[e] * f_base[e];
                    qh[e] = qa[e] * f_base[e];
                    kb[e] = kf[e] * eNL;
                    kc[e] = kb[e] * f_tot[e];                     // k e^{base_{w+1} - Gamma}
                    kh[i][e] = kc[e] * f_hat[e];                  // k e^{Gamma_C - Gamma}
                    t2[e] = kc[e] * f_b2[e];
                    t3[e] = kc[e] * f_b3[e];
                }
                auto put = [&](char* base, const float* f) {
                    *reinterpret_cast<uint2*>(base + offw[i][0]) = pack4_bf16(f[0], f[1], f[2], f[3]);
                    *reinterpret_cast<uint2*>(base + offw[i][1]) = pack4_bf16(f[4], f[5], f[6], f[7]);
                };
                put(kablk + SCR_KA, ka);
                put(kablk + SCR_QA, qa);
                put(rowblk + OFF_KG, kg);
                put(rowblk + OFF_QH, qh);
                put(scr + SCR_BT + bt(w, w) * 4096, kb);
                if (w <= 2) put(scr + SCR_BT + bt(w + 1, w) * 4096, kc);
                if (w <= 1) put(scr + SCR_BT + bt(w + 2, w) * 4096, t2);
                if (w == 0) put(scr + SCR_BT + bt(3, 0) * 4096, t3);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e)
                *reinterpret_cast<uint2*>(smem + OFF_KHT + offkht[e]) =
                    pack4_bf16(kh[0][e], kh[1][e], kh[2][e], kh[3][e]);
            // V^T and beta
            if (tid < 16 * CB) {
                const int rq = tid / CB, cb = tid % CB;
                float vf[4][8];
#pragma unroll
                for (int i = 0; i < 4; ++i) unpack8(keep_if(4 * rq + i < rows, R.v[i]), vf[i]);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    *reinterpret_cast<uint2*>(smem + OFF_VT + vt_off(8 * cb + e, rq)) =
                        pack4_bf16(vf[0][e], vf[1][e], vf[2][e], vf[3][e]);
            }
            if (w == 0) sBeta[lane] = lane < rows ? bf16_bits_to_f32(R.beta) : 0.f;
        }
        __syncthreads();   // (2) phase-A operands visible

        // prefetch the next chunk into registers; consumed one iteration later
        if (ci + 1 < nchunks) {
            const int64_t left1 = left - kC;
            load_chunk<BV>(R, a, tok0 + kC, (int)(left1 < kC ? left1 : kC), h, vt, w, tid);
        }

        // ================= A3: M and P tiles ==================================
        // wave w: M row block w (tiles I <= w) and P row block 3-w (tiles I <= 3-w).
        // Operands are swapped (B tile as A) so the result is the transposed
        // tile: lane (li, lg) holds row li, columns 4lg..4lg+3.
        f32x4 macc[4], pacc[4];
        const int RP = 3 - w;
        {
            bf16x8 af[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) af[kk] = lds_frag(scr + SCR_KA + 16 * w * 256, offA256[kk]);
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                macc[I] = zero4();
                if (I <= w) {
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        macc[I] = mfma_bf16(lds_frag(scr + SCR_BT + bt(w, I) * 4096, offA256[kk]), af[kk], macc[I]);
                }
            }
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) af[kk] = lds_frag(scr + SCR_QA + 16 * RP * 256, offA256[kk]);
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                pacc[I] = zero4();
                if (I <= RP) {
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        pacc[I] = mfma_bf16(lds_frag(scr + SCR_BT + bt(RP, I) * 4096, offA256[kk]), af[kk], pacc[I]);
                }
            }
        }
        __syncthreads();   // (3) operand scratch fully read; MF/TF may overwrite it

        {
            const int rM = 16 * w + li;
            const float bM = sBeta[rM];
            const int rP = 16 * RP + li;
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                if (I <= w) {
                    f32x4 m4;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int i = 16 * I + 4 * lg + j;
                        m4[j] = (i < rM) ? bM * macc[I][j] : 0.f;
                    }
                    *reinterpret_cast<f32x4*>(sMF + rM * FST + 16 * I + 4 * lg) = m4;
                }
                if (I <= RP) {
                    float p[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) p[j] = (16 * I + 4 * lg + j <= rP) ? pacc[I][j] : 0.f;
                    // logical columns 16I+4lg..+3 sit at 4 consecutive positions
                    const int chunk = 4 * (I >> 1) + lg;
                    *reinterpret_cast<uint2*>(smem + OFF_PP + a128(rP, chunk) + 8 * (I & 1)) =
                        pack4_bf16(p[0], p[1], p[2], p[3]);
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
                    const int row = 16 * w + r, col = 16 * w + li;
                    sTF[row * FST + col] = t[r];
                    // logical column col sits at position perm32(col % 32) of its 32-block
                    const int p = 32 * (col >> 5) + perm32(col & 31);
                    *reinterpret_cast<uint16_t*>(smem + OFF_TT + a128(row, p >> 3) + ((p & 7) << 1)) =
                        f32_to_bf16_bits(t[r]);
                }
            }
        }
#pragma unroll
        for (int d = 1; d < 4; ++d) {
            __syncthreads();   // (5,6,7) blocks of the previous level visible
            if (w < 4 - d) {
                const int Rb = w + d, Ib = w;
                // Z = sum_J M_RJ T_JI  (lane holds Z[4lg+j][li])
                f32x4 z = zero4();
                for (int J = Ib; J < Rb; ++J) {
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        z = mfma_f32(sMF[(16 * Rb + li) * FST + 16 * J + 4 * lg + s],
                                     sTF[(16 * J + 4 * lg + s) * FST + 16 * Ib + li], z);
                }
                // (T_RR Z)^T = Z^T T_RR^T: lane holds T_RI[li][4lg+j] after negation
                f32x4 tr = zero4();
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    tr = mfma_f32(z[s], sTF[(16 * Rb + li) * FST + 16 * Rb + 4 * lg + s], tr);
                const int row = 16 * Rb + li;
                *reinterpret_cast<f32x4*>(sTF + row * FST + 16 * Ib + 4 * lg) = -tr;
                const int chunk = 4 * (Ib >> 1) + lg;
                *reinterpret_cast<uint2*>(smem + OFF_TT + a128(row, chunk) + 8 * (Ib & 1)) =
                    pack4_bf16(-tr[0], -tr[1], -tr[2], -tr[3]);
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

            // Y = (gamma K) S (rows t) and O^T = ((gamma Q) S)^T (lane holds 4 columns of row t)
            f32x4 y[4][NCT], ot[4][NCT];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    y[rt][ct] = zero4();
                    ot[rt][ct] = zero4();
                }
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const bf16x8 ak = lds_frag(smem + OFF_KG + rt * 4096, offA256[kk]);
                    const bf16x8 aq = lds_frag(smem + OFF_QH + rt * 4096, offA256[kk]);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        y[rt][ct] = mfma_bf16(ak, sb[kk][ct], y[rt][ct]);
                        ot[rt][ct] = mfma_bf16(sb[kk][ct], aq, ot[rt][ct]);
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
                    const bf16x8 at = lds_frag(smem + OFF_TT + rt * 2048, offA128[kk]);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) u[rt][ct] = mfma_bf16(at, xb[kk][ct], u[rt][ct]);
                }
            }
            bf16x8 ub[2][NCT];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) ub[kk][ct] = pack_frag(u[2 * kk][ct], u[2 * kk + 1][ct]);
            // O^T += (P U)^T, then each lane stores 4 consecutive bf16 of its row
            uint16_t* const o = static_cast<uint16_t*>(a.o);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
                for (int kk = 0; kk <= (rt >> 1); ++kk) {
                    const bf16x8 ap = lds_frag(smem + OFF_PP + rt * 2048, offA128[kk]);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) ot[rt][ct] = mfma_bf16(ub[kk][ct], ap, ot[rt][ct]);
                }
                const int r = 16 * rt + li;
                if (r < rows) {
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) {
                        const f32x4 v4 = a.scale * ot[rt][ct];
                        *reinterpret_cast<uint2*>(o + ((tok0 + r) * a.H + h) * kDV + vt * BV + cw + 16 * ct + 4 * lg) =
                            pack4_bf16(v4[0], v4[1], v4[2], v4[3]);
                    }
                }
            }
            // S <- Diag(e^{Gamma_C}) S + (e^{Gamma_C - Gamma} K)^T U
#pragma unroll
            for (int rt = 0; rt < 8; ++rt) {
                const f32x4 eg = *reinterpret_cast<const f32x4*>(sEgn + 16 * rt + 4 * lg);
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) S[rt][ct] *= eg;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const bf16x8 ah = lds_frag(smem + OFF_KHT + rt * 2048, offKH[kk][rt & 3]);
#pragma unroll
                    for (int ct = 0; ct < NCT; ++ct) S[rt][ct] = mfma_bf16(ah, ub[kk][ct], S[rt][ct]);
                }
            }
        }
    }

    if (a.sT) {
        float* stage = reinterpret_cast<float*>(scr);          // [128][BV] f32
        __syncthreads();
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int j = 0; j < 4; ++j) stage[(16 * rt + 4 * lg + j) * BV + cw + 16 * ct + li] = S[rt][ct][j];
        __syncthreads();
        for (int it = tid; it < kDK * BV / 4; it += kThreads) {
            const int r = it / (BV / 4), c4 = it % (BV / 4);
            *reinterpret_cast<f32x4*>(a.sT + state_base + (int64_t)r * kDV + vt * BV + 4 * c4) =
                *reinterpret_cast<const f32x4*>(stage + r * BV + 4 * c4);
        }
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
