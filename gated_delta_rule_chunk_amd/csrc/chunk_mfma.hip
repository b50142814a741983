// Fused chunkwise KDA forward for bf16 inputs, d_k = d_v = 128, on the
// gfx950 matrix cores.
//
// Per chunk of 16 rows with entry state S (Gamma = in-chunk cumulative
// log-decay per channel; with g >= -5, |Gamma| <= 80 < ln(FLT_MAX), so one
// reference point per chunk suffices):
//   Kg = e^{Gamma} * K,  Qh = e^{Gamma} * Q,  Kb = e^{-Gamma} * K,
//   Kh = e^{Gamma_C - Gamma} * K
//   M = strictly-lower(Diag(beta) Kg Kb^T),  P = lower(Qh Kb^T)
//   T = (I + M)^{-1}        (forward substitution, fp32)
//   U = T Diag(beta) (V - Kg S)
//   O = scale (Qh S + P U)
//   S <- Diag(e^{Gamma_C}) S + Kh^T U
// This is the WY/UT-transform chunk form of the gated delta rule with a
// per-channel decay.
//
// Structure. A workgroup owns one (sequence, head, 64-column half of d_v) and
// runs two kinds of wave side by side, three per SIMD:
//   8 preparation waves, two per chunk of a group of 4: the wave for channel
//     half h of chunk a builds, for channels 64h..64h+63, everything that
//     does not depend on the state (Kg, Qh and Kh^T fragments, e^{Gamma_C},
//     its share of M and P) and stores it to chunk a's slot of an LDS double
//     buffer;
//   4 state waves: wave b carries the fp32 state columns 16b..16b+15 of the
//     half (128 x 16, in registers) through the chunks of the previous group.
//     After that, wave b waits for the two shares of M and P of chunk b of
//     the group being prepared, and forms its T Diag(beta) and -P.
// One barrier per group hands a filled buffer to the state waves and a free
// one to the preparation waves, so preparation of group i+1 overlaps the
// state chain of group i.
//
// Lane layouts. For a 16x16xK matrix-core product an "operand" fragment puts
// the row (A) or column (B) on lane%16 and the contraction slots on lane/16;
// the accumulator ("D") puts rows 4*(lane/16)+j and column lane%16 in a lane.
// Swapping the two operands of a product yields its transpose. A product
// with an identity block (exact for bf16 values) moves data between the two
// layouts; the cumulative decay is a product with a triangular block of ones.
// Accumulator chains never mix the 16x16x32 and 16x16x16 shapes (the
// compiler does not insert enough wait states between the two on gfx950).
//
// Channel order. Preparation works on tiles t = 0..7 of 16 channels: lane
// (li, lg) holds token li and channels 16t + 4lg + j. A 16x16x32 operand
// fragment kk packs tiles 2kk and 2kk+1, so its slot s of lane group lg is
// channel 32kk + 16(s/4) + 4lg + s%4. State tile rt row r is channel 16rt + r,
// so the packed state uses the same slot order.
#include "device_common.hpp"
#include "launchers.hpp"

namespace kda {
namespace {

constexpr int kC = 16;          // rows per chunk
constexpr int kDK = 128;
constexpr int kDV = 128;
constexpr int kNA = 4;          // chunks per group
constexpr int kNP = 2 * kNA;    // preparation waves: two channel halves per chunk
constexpr int kNB = 4;          // state waves, 16 value columns each
constexpr int kBV = 16 * kNB;   // value columns per workgroup
constexpr int kNVT = kDV / kBV;
constexpr int kThreads = 64 * (kNP + kNB);

// One chunk's slot (bytes). Fragments are stored in lane order, so every
// access is 64 consecutive 8- or 16-byte pieces.
constexpr int S_KG = 0;         // [4 kk][64 lanes] bf16x8  (e^G K) operand fragments
constexpr int S_QH = 4096;      // [4 kk][64 lanes] bf16x8  (e^G Q)
constexpr int S_KH = 8192;      // [8 rt][64 lanes] bf16x4  (e^{Gc-G} K)^T, A operand of the state update
constexpr int S_TT = 12288;     // [64 lanes] bf16x4        T Diag(beta), row li, columns 4lg+j
constexpr int S_PN = 12800;     // [64 lanes] bf16x4        -P, row li, columns 4lg+j
constexpr int S_EG = 13312;     // [4 lg][36] f32: entry 4t+j is e^{Gamma_C} of channel 16t+4lg+j
constexpr int EG_STRIDE = 36;   //   (32 used; the pad keeps the lane groups in different banks)
constexpr int SLOT = S_EG + 4 * 4 * EG_STRIDE;
constexpr int S_XP = 2 * kNA * SLOT;            // [buffer][chunk][half]: share of M, P (32 B per lane)
constexpr int S_FS = S_XP + 2 * kNA * 2 * 2048; // per state wave: [16][16] f32 (row-wise N)
constexpr int S_JUNK = S_FS + kNB * 1024;       // per preparation wave: 1 KiB sink for masked-off stores
constexpr int S_FLAG = S_JUNK + kNP * 1024;     // per (chunk, half): int, group + 1 once its share is stored
constexpr int LDS_BYTES = S_FLAG + 4 * kNP;
static_assert(LDS_BYTES <= 163840, "LDS budget");

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8 pack_pair(const f32x4& lo, const f32x4& hi) {
    const bf16x8 r = {(__bf16)lo[0], (__bf16)lo[1], (__bf16)lo[2], (__bf16)lo[3],
                      (__bf16)hi[0], (__bf16)hi[1], (__bf16)hi[2], (__bf16)hi[3]};
    return r;
}
__device__ __forceinline__ bf16x8 pack_pair_neg(const f32x4& lo, const f32x4& hi) {
    const bf16x8 r = {(__bf16)(-lo[0]), (__bf16)(-lo[1]), (__bf16)(-lo[2]), (__bf16)(-lo[3]),
                      (__bf16)(-hi[0]), (__bf16)(-hi[1]), (__bf16)(-hi[2]), (__bf16)(-hi[3])};
    return r;
}
// (two paired conversions; a four-element construction compiles to four
// single conversions and two permutes)
__device__ __forceinline__ bf16x4 pack4v(const f32x4& x) {
    typedef uint32_t u32x2_ __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(bf16x4, u32x2_{pack2_bf16(x[0], x[1]), pack2_bf16(x[2], x[3])});
}
// a 16x16x16 operand widened to a 16x16x32 one: slots 0..3 carry it, 4..7 are zero
__device__ __forceinline__ bf16x8 widen(const bf16x4& x) {
    const __bf16 z = (__bf16)0.f;
    const bf16x8 r = {x[0], x[1], x[2], x[3], z, z, z, z};
    return r;
}
__device__ __forceinline__ f32x4 mfma32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Workgroup barrier that the instruction scheduler may not move work across:
// otherwise it pulls register-only work of the next step (which consumes the
// prefetch just issued) above the barrier and the wave waits for that
// prefetch to land.
__device__ __forceinline__ void group_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
}

// value of x in lane N of this lane's 16-lane row
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + N, 0xf, 0xf, true));
}

// Forward substitution for T = (I + N)^{-1}, N strictly lower triangular.
// Lane (li, lg) holds row li of T in columns 4lg..4lg+3 and the whole row li
// of N in nrow. Eliminating column J: every row i subtracts N[i][J] times the
// (final) row J, which lane (J, lg) of the same 16-lane row holds.
template <int J>
__device__ __forceinline__ void fsub(f32x4& t, const float* nrow) {
    if constexpr (J < 15) {
#pragma unroll
        for (int c = 0; c < 4; ++c) t[c] = fmaf(-nrow[J], row_bcast<J>(t[c]), t[c]);
        fsub<J + 1>(t, nrow);
    }
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// D[rt] = Diag(e) S[rt] for tiles RT..7. e2 holds decay entries 2li, 2li+1
// of this lane's row group; row 4lg+j of tile RT needs entry 4RT+j, held by
// lane 2RT + j/2 of the same 16-lane row.
template <int RT>
__device__ __forceinline__ void decay_state(f32x4 (&D)[8], const f32x4 (&S)[8], const f32x2& e2) {
    if constexpr (RT < 8) {
        D[RT] = f32x4{S[RT][0] * row_bcast<2 * RT>(e2[0]), S[RT][1] * row_bcast<2 * RT>(e2[1]),
                      S[RT][2] * row_bcast<2 * RT + 1>(e2[0]), S[RT][3] * row_bcast<2 * RT + 1>(e2[1])};
        decay_state<RT + 1>(D, S, e2);
    }
}

// Block index -> work item: the two column halves of one (sequence, head) land
// on the same XCD (blocks are dealt round-robin over the 8 XCDs) and are
// dispatched together, so that XCD's L2 serves their shared q, k, g once.
__device__ __forceinline__ int remap_block(int b, int units) {
    const int per = 8 * kNVT;
    const int full = (units / 8) * per;
    if (b >= full) return b;
    const int grp = b / per, rem = b % per;
    return (grp * 8 + (rem & 7)) * kNVT + (rem >> 3);
}

// Buffer descriptors: accesses outside [base, base + num_records) read 0 and
// writes outside it are dropped by the hardware. Rows past a sequence's end
// therefore read as zero tokens (an exact identity step of the recurrence)
// and their outputs are never written, with no branch.
//
// A per-(sequence, head) tensor stream walked one group of 64 rows at a time:
// p is the byte address of the current group's first row (this head's slice),
// rem the bytes from there to the sequence end. The descriptor of a group is
// rebuilt from these with a constant stride; rows within the group are
// addressed through the per-lane offset.
struct Stream {
    const char* p;
    int64_t rem;
};
__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc(const Stream& st) {
    // clamp rem to [0, 2^31 - 1] with 32-bit scalar operations
    const int32_t hi = (int32_t)(st.rem >> 32);
    const uint32_t lo = (uint32_t)st.rem;
    const int32_t n = hi < 0 ? 0 : ((hi > 0 || lo > 0x7fffffffu) ? 0x7fffffff : (int32_t)lo);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(st.p), 0, n, 0x00020000);
}
__device__ __forceinline__ void stream_advance(Stream& st, int64_t bytes) {
    st.p += bytes;
    st.rem -= bytes;
}

struct PrepRegs {
    uint4 q[2], k[2], g[2];   // row li, channels 32(2h+m)+8lg..+7, m = 0, 1
};

// Loads of channel half h of one 16-row chunk for a preparation wave from the
// q, k, g streams positioned at the chunk's group. voff = (16*a + li)*H*256 +
// 128*h + 16*lg bytes for chunk a of the group.
__device__ __forceinline__ void load_prep(PrepRegs& R, const Stream& sq, const Stream& sk, const Stream& sg,
                                          int voff) {
    const __amdgpu_buffer_rsrc_t rq = stream_rsrc(sq);
    const __amdgpu_buffer_rsrc_t rk = stream_rsrc(sk);
    const __amdgpu_buffer_rsrc_t rg = stream_rsrc(sg);
    // issue order = consumption order; memory operations complete in order
#pragma unroll
    for (int m = 0; m < 2; ++m)
        R.g[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rg, voff + 64 * m, 0, 0));
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        R.k[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, voff + 64 * m, 0, 0));
        R.q[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, voff + 64 * m, 0, 0));
    }
}

// ---------------------------------------------------------------------------
// preparation of channel half H of one chunk (wave-local; lane = (li, lg));
// fragments kk = 2H, 2H+1, tiles t = 4H..4H+3
// ---------------------------------------------------------------------------
template <int H>
__device__ __forceinline__ void prepare_half(const PrepRegs& R, char* slot, char* xp, int* flag, int epoch, char* junk,
                                             int li, int lg,
                                             const bf16x8 (&eyeN)[2], const bf16x8 (&eyeP)[2], const bf16x4& lowT) {
    const int lane = li + 16 * lg;
    bf16x8 KA[2], QA[2], KB[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int kk = 2 * H + m;
        const bf16x8 gop = __builtin_bit_cast(bf16x8, R.g[m]);
        const bf16x8 kop = __builtin_bit_cast(bf16x8, R.k[m]);
        const bf16x8 qop = __builtin_bit_cast(bf16x8, R.q[m]);
        f32x4 ka[2], qa[2], kb[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int t = 2 * kk + hf;
            // g^T tile (channel 16t+li, tokens 4lg+j), then Gamma = L * g on
            // the matrix cores: lane gets Gamma[token li][channel 16t+4lg+j]
            const f32x4 gT = mfma32(gop, eyeN[hf], zero4());
            const f32x4 gam = mfma16(pack4v(gT), lowT, zero4());
            // k, q of the same (token, channel) as fp32, by identity products
            const f32x4 kf = mfma32(eyeN[hf], kop, zero4());
            const f32x4 qf = mfma32(eyeN[hf], qop, zero4());
            f32x4 el;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float x = gam[j] * kLog2e;
                el[j] = __builtin_amdgcn_exp2f(x);
                const float enl = __builtin_amdgcn_exp2f(-x);
                ka[hf][j] = kf[j] * el[j];
                qa[hf][j] = qf[j] * el[j];
                kb[hf][j] = kf[j] * enl;
            }
            // token 15 carries e^{Gamma_C}; the other lanes store to the sink
            // (a store under an exec mask would split the schedule)
            *reinterpret_cast<f32x4*>(li == 15 ? slot + S_EG + 4 * (EG_STRIDE * lg + 4 * t) : junk) = el;
        }
        KA[m] = pack_pair(ka[0], ka[1]);
        QA[m] = pack_pair(qa[0], qa[1]);
        KB[m] = pack_pair(kb[0], kb[1]);
        *reinterpret_cast<bf16x8*>(slot + S_KG + 16 * (64 * kk + lane)) = KA[m];
        *reinterpret_cast<bf16x8*>(slot + S_QH + 16 * (64 * kk + lane)) = QA[m];
    }

    // this half's share of M and P, row li, columns 4lg+j
    f32x4 Mr = zero4(), Pr = zero4();
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        Mr = mfma32(KB[m], KA[m], Mr);    // (Kg Kb^T)[li][4lg+j] over these channels
        Pr = mfma32(KB[m], QA[m], Pr);    // (Qh Kb^T)[li][4lg+j]
    }
    *reinterpret_cast<f32x4*>(xp + 32 * lane) = Mr;
    *reinterpret_cast<f32x4*>(xp + 32 * lane + 16) = Pr;
    __hip_atomic_store(flag, epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);

    // (e^{Gamma_C - Gamma} K)^T per state tile: transpose Kb on the matrix
    // cores, then scale channel 16t+li by e^{Gamma_C}
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int t = 4 * H + 2 * m + hf;
            const f32x4 kbT = mfma32(KB[m], eyeP[hf], zero4());   // Kb[token 4lg+j][channel 16t+li]
            const float egc = *reinterpret_cast<const float*>(slot + S_EG + 4 * (EG_STRIDE * (li >> 2) + 4 * t + (li & 3)));
            *reinterpret_cast<bf16x4*>(slot + S_KH + 8 * (64 * t + lane)) = pack4v(kbT * egc);
        }
    }
}

// T Diag(beta) and -P of one chunk from the two halves' shares of M and P
// (wave-local; lane = (li, lg)); fs is this wave's 1 KiB scratch.
__device__ __forceinline__ void finish_chunk(const char* xp, uint32_t beta_bits, char* slot, char* fs, int li, int lg) {
    const int lane = li + 16 * lg;
    const f32x4 Mr = *reinterpret_cast<const f32x4*>(xp + 32 * lane) +
                     *reinterpret_cast<const f32x4*>(xp + 2048 + 32 * lane);
    const f32x4 Pr = *reinterpret_cast<const f32x4*>(xp + 32 * lane + 16) +
                     *reinterpret_cast<const f32x4*>(xp + 2048 + 32 * lane + 16);
    const float beta_li = bf16_bits_to_f32(beta_bits);
    f32x4 bj;   // beta of rows 4lg+j
#pragma unroll
    for (int j = 0; j < 4; ++j) bj[j] = __shfl(beta_li, 4 * lg + j);
    f32x4 Nr, Pn, Tr;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int col = 4 * lg + j;
        Nr[j] = (col < li) ? beta_li * Mr[j] : 0.f;
        Pn[j] = (col <= li) ? -Pr[j] : 0.f;
        Tr[j] = (col == li) ? 1.f : 0.f;
    }
    // T = (I + N)^{-1}: each lane needs its whole row of N
    *reinterpret_cast<f32x4*>(fs + 4 * (16 * li + 4 * lg)) = Nr;
    float nrow[16];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(fs + 4 * (16 * li + 4 * p));
        nrow[4 * p] = x[0]; nrow[4 * p + 1] = x[1]; nrow[4 * p + 2] = x[2]; nrow[4 * p + 3] = x[3];
    }
    fsub<0>(Tr, nrow);
    *reinterpret_cast<bf16x4*>(slot + S_TT + 8 * lane) = pack4v(Tr * bj);
    *reinterpret_cast<bf16x4*>(slot + S_PN + 8 * lane) = pack4v(Pn);
}

__global__ __launch_bounds__(kThreads, 1) void chunk_mfma_kernel(ChunkArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
    const int lane = tid & 63, li = lane & 15, lg = lane >> 4;
    const int units = a.N * a.H;

    // ---- work item ----------------------------------------------------------
    const int wi = remap_block(blockIdx.x, units);
    const int unit = wi / kNVT, vt = wi % kNVT;
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
    const int ngroups = (nchunks + kNA - 1) / kNA;
    const int64_t state_base = ((int64_t)n * a.H + h) * kDK * kDV;
    // hand-over flags start below every step count (LDS holds stale data)
    if (tid < kNP) reinterpret_cast<int*>(smem + S_FLAG)[tid] = 0;
    __syncthreads();

    if (w >= kNB) {
        // ======================= preparation wave ============================
        const int pa = (w - kNB) & (kNA - 1);        // chunk within the group
        const int ph = (w - kNB) / kNA;              // channel half (wave-uniform)
        // the upper half's share of M and P is the last input of the state
        // waves' T: it issues ahead of the lower half
        if (ph == 1) __builtin_amdgcn_s_setprio(1);
        bf16x8 eyeN[2], eyeP[2];   // identity blocks for the natural / packed slot orders
        bf16x4 lowT;               // (L^T)[4lg+s][li] = (4lg+s <= li)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                eyeN[hf][s] = (__bf16)((8 * lg + s == 16 * hf + li) ? 1.f : 0.f);
                eyeP[hf][s] = (__bf16)((s / 4 == hf && 4 * lg + (s & 3) == li) ? 1.f : 0.f);
            }
#pragma unroll
        for (int s = 0; s < 4; ++s) lowT[s] = (__bf16)((4 * lg + s <= li) ? 1.f : 0.f);
        const int64_t row_bytes = (int64_t)a.H * (kDK * 2);          // one token of q, k or g
        const int64_t gstride = (int64_t)kNA * kC * row_bytes;        // one group
        const int64_t head0 = (tok_base * a.H + h) * (int64_t)(kDK * 2);
        Stream sq{static_cast<const char*>(a.q) + head0, len * row_bytes};
        Stream sk{static_cast<const char*>(a.k) + head0, len * row_bytes};
        Stream sg{static_cast<const char*>(a.g) + head0, len * row_bytes};
        const int voff = (kC * pa + li) * (int)row_bytes + 128 * ph + 16 * lg;
        char* const junk = smem + S_JUNK + 1024 * (w - kNB) + 16 * lane;
        int* const flag = reinterpret_cast<int*>(smem + S_FLAG) + 2 * pa + ph;
        // Two register sets alternate (the loop is unrolled by two), so a
        // prefetch is never copied (a copy would wait for it to land). Every
        // step issues its prefetch unconditionally: past the sequence end the
        // buffer range is empty and the loads return zeros without touching
        // memory, and every path through the loop then has the same number of
        // loads in flight, which keeps the compiler's waits exact.
        PrepRegs R0, R1;
        auto step = [&](int it, const PrepRegs& cur, PrepRegs& nxt) {
            load_prep(nxt, sq, sk, sg, voff);            // the streams stand at group it+1
            stream_advance(sq, gstride);
            stream_advance(sk, gstride);
            stream_advance(sg, gstride);
            char* const slot = smem + ((it & 1) * kNA + pa) * SLOT;
            char* const xp = smem + S_XP + (((it & 1) * kNA + pa) * 2 + ph) * 2048;
            if (ph == 0)
                prepare_half<0>(cur, slot, xp, flag, it + 1, junk, li, lg, eyeN, eyeP, lowT);
            else
                prepare_half<1>(cur, slot, xp, flag, it + 1, junk, li, lg, eyeN, eyeP, lowT);
            group_barrier();
        };
        load_prep(R0, sq, sk, sg, voff);
        stream_advance(sq, gstride);
        stream_advance(sk, gstride);
        stream_advance(sg, gstride);
        int it = 0;
        for (; it + 1 < ngroups; it += 2) {
            step(it, R0, R1);
            step(it + 1, R1, R0);
        }
        if (it < ngroups) step(it, R0, R1);
        group_barrier();   // the state waves' last group
    } else {
        // ========================== state wave ===============================
        // The state chain is the serial critical path: its waves issue first,
        // and the preparation waves fill the issue slots it leaves idle.
        __builtin_amdgcn_s_setprio(2);
        const int cw = 16 * w;                       // this wave's columns within the half
        const int col0 = vt * kBV + cw;              // ... within d_v
        f32x4 S[8];                                  // tile rt: [channel 16rt+4lg+j][column col0+li]
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                S[rt][j] = a.s0 ? a.s0[state_base + (int64_t)(16 * rt + 4 * lg + j) * kDV + col0 + li] : 0.f;

        bf16x8 eyeV;   // [slot 8lg+s][column li] = (s < 4 && 4lg+s == li)
#pragma unroll
        for (int s = 0; s < 8; ++s) eyeV[s] = (__bf16)((s < 4 && 4 * lg + s == li) ? 1.f : 0.f);
        const float neg_scale = -a.scale;

        // Value tiles of group gi and beta of this wave's chunk of group gi+1
        // (used one iteration later, like the tiles): two register sets
        // alternate and the loads are unconditional, as in the preparation
        // waves.
        const int64_t vrow_bytes = (int64_t)a.H * (kDV * 2);          // one token of v or o
        const int64_t head0 = (tok_base * a.H + h) * (int64_t)(kDV * 2) + col0 * 2;
        Stream sv{static_cast<const char*>(a.v) + head0, len * vrow_bytes - col0 * 2};
        Stream so{static_cast<const char*>(a.o) + head0, len * vrow_bytes - col0 * 2};
        Stream sb{static_cast<const char*>(a.beta) + (tok_base * a.H + h) * 2, len * a.H * 2};
        const int64_t vstride = (int64_t)kNA * kC * vrow_bytes, bstride = (int64_t)kNA * kC * a.H * 2;
        int vofs[kNA];                                 // row li of chunk s, columns 4lg..4lg+3
#pragma unroll
        for (int s = 0; s < kNA; ++s) vofs[s] = (kC * s + li) * (int)vrow_bytes + 8 * lg;
        const int voffb = (kC * w + li) * a.H * 2;     // beta of row li of this wave's chunk
        char* const fs = smem + S_FS + 1024 * w;
        int* const flags = reinterpret_cast<int*>(smem + S_FLAG);
        // (one vector value per set: an array here would be left in private
        // memory, and every prefetch would then wait to be stored there)
        struct StateIn { u32x8 v; uint32_t beta; };   // tile s in v[2s], v[2s+1]
        StateIn VA, VB;
        // sv stands at group gi, sb at group gi+1 when group gi is loaded
        auto load_group = [&](StateIn& in) {
            in.beta = __builtin_amdgcn_raw_buffer_load_b16(stream_rsrc(sb), voffb, 0, 0);
            const __amdgpu_buffer_rsrc_t rv = stream_rsrc(sv);
#pragma unroll
            for (int s = 0; s < kNA; ++s) {
                const u32x2 t = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rv, vofs[s], 0, 0));
                in.v[2 * s] = t[0];
                in.v[2 * s + 1] = t[1];
            }
            stream_advance(sv, vstride);
            stream_advance(sb, bstride);
        };
        // Chunks of group gi from its LDS buffer. Unconditional: a chunk past
        // the sequence end holds zero tokens, which leave the state unchanged,
        // and its output stores fall outside the store buffer's range, so the
        // hardware drops them.
        // T Diag(beta) and -P of chunk w of group gi, once both preparation
        // halves have stored their shares (bounded wait: they store them every
        // step before the barrier, so they always arrive)
        auto finish = [&](int gi, uint32_t beta_bits) {
            for (int spin = 0; spin < (1 << 22); ++spin) {
                if (__hip_atomic_load(flags + 2 * w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == gi + 1 &&
                    __hip_atomic_load(flags + 2 * w + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == gi + 1)
                    break;
                __builtin_amdgcn_s_sleep(1);
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            finish_chunk(smem + S_XP + ((gi & 1) * kNA + w) * 4096, beta_bits,
                         smem + ((gi & 1) * kNA + w) * SLOT, fs, li, lg);
        };
        // so stands at group gi when group gi is consumed
        auto consume = [&](int gi, const StateIn& vcur) {
            const __amdgpu_buffer_rsrc_t ro = stream_rsrc(so);
            stream_advance(so, vstride);
#pragma unroll
            for (int s = 0; s < kNA; ++s) {
                const char* const slot = smem + ((gi & 1) * kNA + s) * SLOT;
                bf16x8 sbn[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) sbn[kk] = pack_pair_neg(S[2 * kk], S[2 * kk + 1]);
                // decayed state for the update at the end of the chunk. Lane li of
                // row group lg reads entries 2li, 2li+1 of the group's 32 decay
                // factors; DPP broadcasts the one each row needs.
                const f32x2 e2 = *reinterpret_cast<const f32x2*>(slot + S_EG + 4 * (EG_STRIDE * lg + 2 * li));
                f32x4 D[8];
                decay_state<0>(D, S, e2);
                // X = V - Kg S  (rows 4lg+j, column li)
                const bf16x8 vop = widen(__builtin_bit_cast(bf16x4, u32x2{vcur.v[2 * s], vcur.v[2 * s + 1]}));
                f32x4 X = mfma32(vop, eyeV, zero4());
                // OT = -(Qh S)^T  (column 4lg+j of row li)
                f32x4 OT = zero4();
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const bf16x8 kg = *reinterpret_cast<const bf16x8*>(slot + S_KG + 16 * (64 * kk + lane));
                    const bf16x8 qh = *reinterpret_cast<const bf16x8*>(slot + S_QH + 16 * (64 * kk + lane));
                    X = mfma32(kg, sbn[kk], X);
                    OT = mfma32(sbn[kk], qh, OT);
                }
                const bf16x4 tt = *reinterpret_cast<const bf16x4*>(slot + S_TT + 8 * lane);
                const f32x4 U = mfma16(tt, pack4v(X), zero4());      // U[4lg+j][li]
                const bf16x4 ub = pack4v(U);
                const bf16x4 pn = *reinterpret_cast<const bf16x4*>(slot + S_PN + 8 * lane);
                OT = mfma32(widen(ub), widen(pn), OT);               // -(Qh S + P U)^T
                __builtin_amdgcn_raw_buffer_store_b64(
                    u32x2{pack2_bf16(neg_scale * OT[0], neg_scale * OT[1]),
                          pack2_bf16(neg_scale * OT[2], neg_scale * OT[3])},
                    ro, vofs[s], 0, 0);
                // S <- Diag(e^{Gamma_C}) S + Kh^T U (the decayed state D was
                // formed at the top of the chunk, off the critical path)
#pragma unroll
                for (int rt = 0; rt < 8; ++rt) {
                    const bf16x4 kh = *reinterpret_cast<const bf16x4*>(slot + S_KH + 8 * (64 * rt + lane));
                    S[rt] = mfma16(kh, ub, D[rt]);
                }
            }
        };
        // iteration it loads group it, consumes group it-1 and finishes chunk w
        // of group it
        const uint32_t beta0 = __builtin_amdgcn_raw_buffer_load_b16(stream_rsrc(sb), voffb, 0, 0);
        stream_advance(sb, bstride);
        load_group(VA);
        if (ngroups > 0) finish(0, beta0);
        group_barrier();
        int it = 1;
        for (; it + 1 <= ngroups; it += 2) {
            load_group(VB);
            consume(it - 1, VA);
            if (it < ngroups) finish(it, VA.beta);
            group_barrier();
            load_group(VA);
            consume(it, VB);
            if (it + 1 < ngroups) finish(it + 1, VB.beta);
            group_barrier();
        }
        if (it <= ngroups) {
            load_group(VB);
            consume(it - 1, VA);
            if (it < ngroups) finish(it, VA.beta);
            group_barrier();
        }
        if (a.sT) {
#pragma unroll
            for (int rt = 0; rt < 8; ++rt)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    a.sT[state_base + (int64_t)(16 * rt + 4 * lg + j) * kDV + col0 + li] = S[rt][j];
        }
    }
}

}  // namespace

bool chunk_mfma_supported(const ChunkArgs& a) {
    return a.bf16 && a.Dk == kDK && a.Dv == kDV;
}

hipError_t launch_chunk_mfma(const ChunkArgs& a, hipStream_t s) {
    const int units = a.N * a.H;
    hipLaunchKernelGGL(chunk_mfma_kernel, dim3((unsigned)(units * kNVT)), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace kda
