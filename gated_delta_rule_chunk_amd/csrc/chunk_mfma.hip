// Fused chunkwise KDA forward for bf16 inputs, d_k = d_v = 128, on the
// gfx950 matrix cores.
//
// Structure. A workgroup of NW waves owns one (sequence, head, BV = 16*NW
// column slice of d_v) and walks the sequence in groups of NW chunks of 16
// rows. Per group:
//   phase A  wave w builds, alone and entirely in registers, everything that
//            depends only on k, g, beta, q, v of chunk w of the group, and
//            publishes it to its LDS slot;
//   barrier
//   phase B  every wave advances its 16 state columns through the NW chunks
//            in order (the state-dependent chain);
//   barrier.
// The float32 state slice (128 x 16 per wave) never leaves registers.
//
// Per chunk of 16 rows with entry state S (Gamma = in-chunk cumulative
// log-decay per channel; with g >= -5, |Gamma| <= 80 < ln(FLT_MAX), so no
// intermediate reference point is needed inside a chunk):
//   Kg = e^{Gamma} * K,  Qh = e^{Gamma} * Q,  Kb = e^{-Gamma} * K,
//   Kh = e^{Gamma_C - Gamma} * K
//   M = strictly-lower(Diag(beta) Kg Kb^T),  P = lower(Qh Kb^T)
//   T = (I + M)^{-1} = (I - M)(I + M^2)(I + M^4)(I + M^8)   (M^16 = 0),
//       applied as T' = T Diag(beta)
//   U = T' (V - Kg S)
//   O = scale (Qh S + P U)
//   S <- Diag(e^{Gamma_C}) S + Kh^T U
// This is the WY/UT-transform chunk form of the gated delta rule with a
// per-channel decay.
//
// Lane layouts. For the 16x16xK matrix-core products, an "operand" fragment
// puts the row (A) or column (B) on lane%16 and the contraction slots on
// lane/16; a "D" accumulator puts rows 4*(lane/16)+j and column lane%16 in a
// lane. A pair of D tiles holds, per lane group, exactly the 8 contraction
// slots a 16x16x32 operand expects, and one D tile the 4 slots of a
// 16x16x16 operand, so accumulators feed later products with no data
// movement. Swapping the two operands of a product yields its transpose.
// The only hardware facts relied on are: A row / B column = lane%16, A and B
// map their contraction slots per lane group identically, and the D layout
// above. Accumulator chains never mix the 16x16x32 and 16x16x16 shapes. State tile rt row r16 holds d_k index pi(rt, r16) =
// 32*(rt/2) + 8*(r16/4) + 4*(rt%2) + r16%4, so the S operand slots are 8
// consecutive channels and every LDS operand is stored in natural order.
//
// Phase A works in "row" layout: lane (li, lg) holds row li of the chunk and
// the channels 32kk+8lg..+7 (kk = 0..3), which are exactly the operand
// fragments of Kg, Qh, Kb. The cumulative decay is a 16-lane DPP scan. K_h
// and V are turned into the D layout by multiplying with an identity block
// on the matrix cores (exact for bf16 values) before their transposed store.
#include "device_common.hpp"
#include "launchers.hpp"

namespace kda {
namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kC = 16;       // rows per chunk
constexpr int kDK = 128;
constexpr int kDV = 128;

template <int NW>
struct Cfg {
    static constexpr int BV = 16 * NW;          // value columns per workgroup
    static constexpr int THREADS = 64 * NW;
    // one slot per chunk of a group (bytes)
    static constexpr int S_KG = 0;              // [16][128] bf16  e^{G} K      (16-B chunks XOR row)
    static constexpr int S_QH = 4096;           // [16][128] bf16  e^{G} Q
    static constexpr int S_KHT = 8192;          // [128][16] bf16  (e^{Gc-G} K)^T (8-B pieces XOR row/8)
    static constexpr int S_TT = 12288;          // [16][16]  bf16  T Diag(beta)
    static constexpr int S_PP = 12800;          // [16][16]  bf16  P
    static constexpr int S_EGN = 13312;         // [128]     f32   e^{Gamma_C}
    static constexpr int S_VT = 13824;          // [BV][16]  bf16  V^T          (8-B pieces XOR row/8)
    static constexpr int SLOT = S_VT + BV * 32;
    static constexpr int LDS = NW * SLOT;
};
static_assert(Cfg<8>::LDS <= 163840, "LDS budget");
static_assert(Cfg<4>::LDS >= 128 * 64 * 4 && Cfg<8>::LDS >= 128 * 128 * 4, "state staging fits");

__device__ __forceinline__ int pi_row(int rt, int r16) {
    return 32 * (rt >> 1) + 8 * (r16 >> 2) + 4 * (rt & 1) + (r16 & 3);
}
__device__ __forceinline__ int kg_off(int row, int chunk) { return row * 256 + ((chunk ^ row) << 4); }
__device__ __forceinline__ int t32_off(int row, int piece) {   // [rows][16] bf16, 4 pieces of 8 B
    return row * 32 + ((piece ^ ((row >> 3) & 3)) << 3);
}

__device__ __forceinline__ bf16x8 pack8(const float* f) {
    const bf16x8 r = {(__bf16)f[0], (__bf16)f[1], (__bf16)f[2], (__bf16)f[3],
                      (__bf16)f[4], (__bf16)f[5], (__bf16)f[6], (__bf16)f[7]};
    return r;
}
__device__ __forceinline__ bf16x8 pack_pair(const f32x4& lo, const f32x4& hi) {
    const bf16x8 r = {(__bf16)lo[0], (__bf16)lo[1], (__bf16)lo[2], (__bf16)lo[3],
                      (__bf16)hi[0], (__bf16)hi[1], (__bf16)hi[2], (__bf16)hi[3]};
    return r;
}
__device__ __forceinline__ bf16x4 pack4v(const f32x4& x) {
    const bf16x4 r = {(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
    return r;
}
__device__ __forceinline__ f32x4 mfma32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 16x16 products for the inverse. "row" form: lane (li, lg) holds
// X[li][4lg+j]; "col" form: lane holds X[4lg+j][li].
__device__ __forceinline__ f32x4 mm_col(const f32x4& xr, const f32x4& yc) {   // (X Y) col
    f32x4 d = zero4();
#pragma unroll
    for (int s = 0; s < 4; ++s) d = __builtin_amdgcn_mfma_f32_16x16x4f32(xr[s], yc[s], d, 0, 0, 0);
    return d;
}
__device__ __forceinline__ f32x4 mm_row(const f32x4& xr, const f32x4& yc) {   // (X Y) row
    f32x4 d = zero4();
#pragma unroll
    for (int s = 0; s < 4; ++s) d = __builtin_amdgcn_mfma_f32_16x16x4f32(yc[s], xr[s], d, 0, 0, 0);
    return d;
}

// inclusive prefix sum over the 16 lanes of a row (lane%16), zero-filled
__device__ __forceinline__ float scan16(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xf, 0xf, true));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x112, 0xf, 0xf, true));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xf, 0xf, true));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x118, 0xf, 0xf, true));
    return x;
}

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

template <int NW>
struct ChunkRegs {
    uint4 q[4], k[4], g[4];
    uint4 v[NW / 2];      // BV/32 blocks of 32 value columns
    uint32_t beta;        // raw bf16 bits
};

// Buffer resource over [base, base + nbytes): accesses outside it read 0 and
// writes outside it are dropped by the hardware. This is how rows past a
// sequence's end become zero tokens (an exact identity step of the
// recurrence) and how their outputs are never written, with no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t nbytes) {
    const int32_t n = nbytes <= 0 ? 0 : (nbytes > 0x7fffffff ? 0x7fffffff : (int32_t)nbytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

// Loads of one 16-row chunk (sequence rows first..first+15) in row layout:
// lane (li, lg) gets row li, channels 32kk+8lg..+7 and value columns
// 32p+8lg..+7 of its slice. voff = li*H*256 + 16*lg bytes, voffb = li*H*2.
template <int NW>
__device__ __forceinline__ void load_chunk(ChunkRegs<NW>& R, const ChunkArgs& a, int64_t tok_base,
                                           int64_t first, int64_t len, int h, int vt, int voff, int voffb) {
    const int64_t row0 = (tok_base + first) * a.H + h;
    const int64_t span = (len - first) * a.H * (int64_t)(kDK * 2);    // bytes to the sequence end
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(static_cast<const uint16_t*>(a.q) + row0 * kDK, span);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(static_cast<const uint16_t*>(a.k) + row0 * kDK, span);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(static_cast<const uint16_t*>(a.g) + row0 * kDK, span);
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc(static_cast<const uint16_t*>(a.v) + row0 * kDV + vt * Cfg<NW>::BV, span - vt * Cfg<NW>::BV * 2);
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(static_cast<const uint16_t*>(a.beta) + row0, (len - first) * a.H * 2);
    // issue order = roughly consumption order, so each use waits only for
    // the loads it needs (memory operations complete in issue order)
    R.beta = __builtin_amdgcn_raw_buffer_load_b16(rb, voffb, 0, 0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        R.g[kk] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rg, voff + 64 * kk, 0, 0));
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        R.k[kk] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, voff + 64 * kk, 0, 0));
        R.q[kk] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, voff + 64 * kk, 0, 0));
    }
#pragma unroll
    for (int p = 0; p < NW / 2; ++p)
        R.v[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, voff + 64 * p, 0, 0));
}

template <int NW>
__global__ __launch_bounds__(64 * NW, 1) void chunk_mfma_kernel(ChunkArgs a) {
    using CF = Cfg<NW>;
    constexpr int BV = CF::BV;
    constexpr int NVT = kDV / BV;
    __shared__ __attribute__((aligned(16))) char smem[CF::LDS];

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
        int* lens = reinterpret_cast<int*>(smem);
        int* pick = lens + 256;
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
    const int64_t tok_base = b * (int64_t)a.T + bos;          // token index of row 0
    const int nchunks = (int)((len + kC - 1) / kC);
    const int ngroups = (nchunks + NW - 1) / NW;
    const int64_t state_base = ((int64_t)n * a.H + h) * kDK * kDV;
    const int cw = 16 * w;                                    // this wave's slice columns

    // ---- state tiles (wave w: 128 x 16, tile rt row r16 = d_k pi(rt, r16)) ----
    f32x4 S[8];
    if (a.s0) {
        float* stage = reinterpret_cast<float*>(smem);       // [128][BV] f32, coalesced staging
        for (int it = tid; it < kDK * BV / 4; it += CF::THREADS) {
            const int r = it / (BV / 4), c4 = it % (BV / 4);
            *reinterpret_cast<f32x4*>(stage + r * BV + 4 * c4) =
                *reinterpret_cast<const f32x4*>(a.s0 + state_base + (int64_t)r * kDV + vt * BV + 4 * c4);
        }
        __syncthreads();
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int j = 0; j < 4; ++j) S[rt][j] = stage[pi_row(rt, 4 * lg + j) * BV + cw + li];
        __syncthreads();
    } else {
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) S[rt] = zero4();
    }

    // identity halves for the register transposes: slot s of lane group lg is
    // channel 8lg+s of a 32-block; column li of half hf is channel 16hf+li
    bf16x8 eye[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int s = 0; s < 8; ++s) eye[hf][s] = (__bf16)((8 * lg + s == 16 * hf + li) ? 1.f : 0.f);

    const int voff = li * a.H * (kDK * 2) + 16 * lg;          // row li, 8 channels at 8lg
    const int voffb = li * a.H * 2;
    const int voffo = li * a.H * (kDV * 2) + (cw + 4 * lg) * 2;   // output row li, 4 columns
    ChunkRegs<NW> R;
    if (ngroups > 0) load_chunk<NW>(R, a, tok_base, (int64_t)w * kC, len, h, vt, voff, voffb);

    uint16_t* const out = static_cast<uint16_t*>(a.o);
    for (int grp = 0; grp < ngroups; ++grp) {
        // ========== phase A: wave w prepares chunk c = grp*NW + w ==========
        {
            const int c = grp * NW + w;
            char* const slot = smem + w * CF::SLOT;

            // cumulative log2-decay over the 16 rows (DPP scan along lane%16)
            float G[4][8];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                float gf[8];
                unpack8(R.g[kk], gf);
#pragma unroll
                for (int e = 0; e < 8; ++e) G[kk][e] = scan16(gf[e] * kLog2e);
            }
            // decayed operands
            bf16x8 KA[4], QA[4], KB[4];
            float eL15[4][8];   // e^{Gamma} of this lane's channels (row li); row 15 gives e^{Gamma_C}
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                float kf[8], qf[8], ka[8], qa[8], kb[8];
                unpack8(R.k[kk], kf);
                unpack8(R.q[kk], qf);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float el = exp2_fast(G[kk][e]);
                    const float enl = exp2_fast(-G[kk][e]);
                    eL15[kk][e] = el;
                    ka[e] = kf[e] * el;
                    qa[e] = qf[e] * el;
                    kb[e] = kf[e] * enl;
                }
                KA[kk] = pack8(ka);
                QA[kk] = pack8(qa);
                KB[kk] = pack8(kb);
                *reinterpret_cast<bf16x8*>(slot + CF::S_KG + kg_off(li, 4 * kk + lg)) = KA[kk];
                *reinterpret_cast<bf16x8*>(slot + CF::S_QH + kg_off(li, 4 * kk + lg)) = QA[kk];
            }
            // e^{Gamma_C} per channel: row 15 publishes, then every lane reads its channels
            if (li == 15) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    *reinterpret_cast<f32x4*>(slot + CF::S_EGN + 4 * (32 * kk + 8 * lg)) =
                        f32x4{eL15[kk][0], eL15[kk][1], eL15[kk][2], eL15[kk][3]};
                    *reinterpret_cast<f32x4*>(slot + CF::S_EGN + 4 * (32 * kk + 8 * lg + 4)) =
                        f32x4{eL15[kk][4], eL15[kk][5], eL15[kk][6], eL15[kk][7]};
                }
            }

            // M (both layouts) and P (row layout): contraction over the 128 channels
            f32x4 Mc = zero4(), Mr = zero4(), Pr = zero4();
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                Mc = mfma32(KA[kk], KB[kk], Mc);    // lane: M[4lg+j][li]
                Mr = mfma32(KB[kk], KA[kk], Mr);    // lane: M[li][4lg+j]
                Pr = mfma32(KB[kk], QA[kk], Pr);    // lane: P[li][4lg+j]
            }
            const float beta_li = bf16_bits_to_f32(R.beta);
            f32x4 bj;   // beta of rows 4lg+j
#pragma unroll
            for (int j = 0; j < 4; ++j) bj[j] = __shfl(beta_li, 4 * lg + j);
            f32x4 Nc, Nr, Id, Pm;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int q4 = 4 * lg + j;
                Nc[j] = (li < q4) ? bj[j] * Mc[j] : 0.f;       // N[q4][li], strictly lower
                Nr[j] = (q4 < li) ? beta_li * Mr[j] : 0.f;     // N[li][q4]
                Pm[j] = (q4 <= li) ? Pr[j] : 0.f;              // P[li][q4], lower incl. diagonal
                Id[j] = (q4 == li) ? 1.f : 0.f;
            }
            // T = (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8)
            const f32x4 N2c = mm_col(Nr, Nc), N2r = mm_row(Nr, Nc);
            const f32x4 N4c = mm_col(N2r, N2c), N4r = mm_row(N2r, N2c);
            const f32x4 N8c = mm_col(N4r, N4c);
            const f32x4 P1r = Id - Nr;
            const f32x4 P2r = P1r + mm_row(P1r, N2c);
            const f32x4 P3r = P2r + mm_row(P2r, N4c);
            const f32x4 Tr = P3r + mm_row(P3r, N8c);           // T[li][4lg+j]
            *reinterpret_cast<bf16x4*>(slot + CF::S_TT + t32_off(li, lg)) = pack4v(Tr * bj);
            *reinterpret_cast<bf16x4*>(slot + CF::S_PP + t32_off(li, lg)) = pack4v(Pm);

            // (e^{Gamma_C - Gamma} K)^T: transpose Kb on the matrix cores, then
            // scale channel by channel with e^{Gamma_C}
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int ch = 32 * kk + 16 * hf + li;
                    const f32x4 kbT = mfma32(KB[kk], eye[hf], zero4());   // Kb[4lg+j][ch]
                    const float egc = *reinterpret_cast<const float*>(slot + CF::S_EGN + 4 * ch);
                    *reinterpret_cast<bf16x4*>(slot + CF::S_KHT + t32_off(ch, lg)) = pack4v(kbT * egc);
                }
            }
            // V^T
#pragma unroll
            for (int p = 0; p < NW / 2; ++p) {
                const bf16x8 vf = __builtin_bit_cast(bf16x8, R.v[p]);
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const f32x4 vT = mfma32(vf, eye[hf], zero4());        // V[4lg+j][32p+16hf+li]
                    *reinterpret_cast<bf16x4*>(slot + CF::S_VT + t32_off(32 * p + 16 * hf + li, lg)) = pack4v(vT);
                }
            }
            // prefetch this wave's chunk of the next group
            if (grp + 1 < ngroups) {
                const int cn = c + NW;
                load_chunk<NW>(R, a, tok_base, (int64_t)cn * kC, len, h, vt, voff, voffb);
            }
        }
        __syncthreads();   // all chunks of the group published

        // ========== phase B: the state chain through the group's chunks ==========
        // Unrolled and unconditional: a chunk past the sequence end holds zero
        // tokens, which leave the state unchanged, and its output stores fall
        // outside the store buffer's range, so the hardware drops them.
#pragma unroll
        for (int s = 0; s < NW; ++s) {
            const int c = grp * NW + s;
            const char* const slot = smem + s * CF::SLOT;
            const __amdgpu_buffer_rsrc_t ro =
                make_rsrc(out + ((tok_base + (int64_t)c * kC) * a.H + h) * kDV + vt * BV,
                          (len - (int64_t)c * kC) * a.H * (kDV * 2) - vt * BV * 2);

            bf16x8 sb[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) sb[kk] = pack_pair(S[2 * kk], S[2 * kk + 1]);
            f32x4 Y = zero4(), OT = zero4();
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const bf16x8 kg = *reinterpret_cast<const bf16x8*>(slot + CF::S_KG + kg_off(li, 4 * kk + lg));
                const bf16x8 qh = *reinterpret_cast<const bf16x8*>(slot + CF::S_QH + kg_off(li, 4 * kk + lg));
                Y = mfma32(kg, sb[kk], Y);       // Y[4lg+j][li]   = (Kg S)[t][n]
                OT = mfma32(sb[kk], qh, OT);     // OT[4lg+j][li]  = (Qh S)[li][4lg+j]
            }
            const bf16x4 vv = *reinterpret_cast<const bf16x4*>(slot + CF::S_VT + t32_off(cw + li, lg));
            f32x4 X;
#pragma unroll
            for (int j = 0; j < 4; ++j) X[j] = (float)vv[j] - Y[j];
            const bf16x4 tt = *reinterpret_cast<const bf16x4*>(slot + CF::S_TT + t32_off(li, lg));
            const f32x4 U = mfma16(tt, pack4v(X), zero4());        // U[4lg+j][li]
            const bf16x4 ub = pack4v(U);
            const bf16x4 pp = *reinterpret_cast<const bf16x4*>(slot + CF::S_PP + t32_off(li, lg));
            // (P U)[li][4lg+j]. Accumulated separately: a 16x16x16 product must not
            // take a 16x16x32 result as its accumulator input (the compiler does not
            // insert enough wait states between the two shapes on gfx950).
            OT += mfma16(ub, pp, zero4());
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            __builtin_amdgcn_raw_buffer_store_b64(
                u32x2{pack2_bf16(a.scale * OT[0], a.scale * OT[1]), pack2_bf16(a.scale * OT[2], a.scale * OT[3])},
                ro, voffo, 0, 0);
            // S <- Diag(e^{Gamma_C}) S + Kh^T U
#pragma unroll
            for (int rt = 0; rt < 8; ++rt) {
                const f32x4 eg = *reinterpret_cast<const f32x4*>(slot + CF::S_EGN + 4 * pi_row(rt, 4 * lg));
                const bf16x4 kh = *reinterpret_cast<const bf16x4*>(slot + CF::S_KHT + t32_off(pi_row(rt, li), lg));
                S[rt] = mfma16(kh, ub, S[rt] * eg);
            }
        }
        __syncthreads();   // slots free for the next group
    }

    if (a.sT) {
        float* stage = reinterpret_cast<float*>(smem);       // [128][BV] f32
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int j = 0; j < 4; ++j) stage[pi_row(rt, 4 * lg + j) * BV + cw + li] = S[rt][j];
        __syncthreads();
        for (int it = tid; it < kDK * BV / 4; it += CF::THREADS) {
            const int r = it / (BV / 4), c4 = it % (BV / 4);
            *reinterpret_cast<f32x4*>(a.sT + state_base + (int64_t)r * kDV + vt * BV + 4 * c4) =
                *reinterpret_cast<const f32x4*>(stage + r * BV + 4 * c4);
        }
    }
}

}  // namespace

bool chunk_mfma_supported(const ChunkArgs& a) {
    return a.bf16 && a.Dk == kDK && a.Dv == kDV;
}

// Slice width: 4 waves x 16 columns (two workgroups per head) while
// (sequences x heads) leaves CUs idle; 8 waves x 16 columns (one workgroup
// per head, no duplicated state-independent work) once there are enough heads.
hipError_t launch_chunk_mfma(const ChunkArgs& a, hipStream_t s) {
    const int units = a.N * a.H;
    if (units <= 256) {
        hipLaunchKernelGGL(chunk_mfma_kernel<4>, dim3((unsigned)(units * 2)), dim3(256), 0, s, a);
    } else {
        hipLaunchKernelGGL(chunk_mfma_kernel<8>, dim3((unsigned)units), dim3(512), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace kda
