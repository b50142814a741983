// Intra-sequence split of the chunk forward: each sequence is cut into P
// segments that run as independent sequences, and the segments are joined by
// the affine form of the state map.
//
// Over one segment the recurrence maps its entry state linearly plus a
// constant: S_out = A S_in + B, where B is the segment's final state from a
// zero entry state and A (d_k x d_k) is its final state from the identity
// with v = 0. The same holds row by row: the state after row t is
// A_t S_in + B_t, so the output of row t is o_B(t) + S_inᵀ (scale A_tᵀ q_t),
// and scale A_tᵀ q_t is the output of the A pass.
//
// bf16, d_k = d_v = 128 (the matrix-core kernel), one call runs:
//   1. one launch over all segments with twice the column blocks: B from a
//      zero entry state (the sequence's initial state in its first segment),
//      writing its outputs into o, and A (segments p >= 1) from the identity
//      with v = 0, writing its outputs scale A_tᵀ q_t into the workspace;
//   2. split_scan_kernel: S_in(1) = B(0), S_in(p) = A(p-1) S_in(p-1) + B(p-1),
//      and the final state A(P-1) S_in(P-1) + B(P-1);
//   3. split_correct_kernel: o += S_in(p)ᵀ (scale A_tᵀ q_t) on the rows of
//      segments p >= 1.
// A first segment runs only B, so it takes two shares of rows and every
// later segment one: each segment then carries the same work.
// Every other shape runs three forward passes: B from zero entry states
// (outputs discarded), A from the identity, the scan from the initial state,
// then the forward over all segments from S_in, which writes o.
// Each forward pass puts P times as many workgroups on the chip as the
// unsplit call.
#include <algorithm>
#include <mutex>

#include <type_traits>

#include "device_common.hpp"
#include "launchers.hpp"

namespace kda {
namespace {

// Segment offsets for every sequence (split_segment's cut) as packed
// cu_seqlens of the N * P segments.
__global__ void split_offsets_kernel(const int32_t* cu, int32_t N, int32_t T, int32_t P, int32_t* seg_cu) {
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    int64_t bos = 0, len = 0;
    for (int p = 0; p < P; ++p) {
        split_segment(cu, T, P, 1, (int64_t)n * P + p, bos, len);
        seg_cu[(int64_t)n * P + p] = (int32_t)bos;
    }
    if (n == N - 1) seg_cu[(int64_t)N * P] = (int32_t)(bos + len);
}

// Identity [Dk][Dk] per (segment, head).
__global__ void fill_identity_kernel(float* p, int64_t mats, int Dk) {
    const int64_t n = mats * Dk * Dk;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const int64_t e = i % ((int64_t)Dk * Dk);
        p[i] = (e / Dk == e % Dk) ? 1.f : 0.f;
    }
}

// One workgroup per (sequence, head, 16-column slice of d_v): the chain of
// entry states S_in(p) over the sequence's P segments, and its final state.
// A is [N*P][H][Dk][Dk], Bst and Sin are [N*P][H][Dk][Dv]. Each step stages
// A(p) in LDS with coalesced 16-byte loads.
template <int DK>
constexpr int scan_threads() { return DK == 128 ? 512 : 256; }
template <int DK>
__global__ __launch_bounds__(scan_threads<DK>()) void split_scan_kernel(const float* A, const float* Bst,
                                                                        const float* s0, float* Sin, float* sT,
                                                                        int32_t N, int32_t H, int32_t Dv, int32_t P) {
    constexpr int BVs = 16;
    constexpr int NT = scan_threads<DK>();
    constexpr int kQuads = DK * DK / 4;                       // float4 pieces of A
    constexpr int kPer = kQuads / NT > 0 ? kQuads / NT : 1;   // per thread
    constexpr int kOut = DK * BVs / NT > 0 ? DK * BVs / NT : 1;
    __shared__ __attribute__((aligned(16))) float sA[DK][DK + 4];
    __shared__ float sS[DK][BVs + 1];
    // DK = 128: S again as bf16 hi and lo parts, transposed ([column][channel]),
    // the B operands of the products
    constexpr int kSplitRows = DK == 128 ? BVs : 1;
    __shared__ __attribute__((aligned(16))) __bf16 sSh[kSplitRows][DK + 8];
    __shared__ __attribute__((aligned(16))) __bf16 sSl[kSplitRows][DK + 8];
    const int tid = threadIdx.x;
    const int nvt = Dv / BVs;
    // blocks are dealt round-robin over the 8 XCDs: the column slices of one
    // (sequence, head), which all read its A(p), go to one XCD so that its L2
    // serves the repeats (the last units, below a multiple of 8, stay spread)
    int b = blockIdx.x;
    {
        const int units = N * H, per = 8 * nvt, full = (units / 8) * per;
        if (b < full) b = (b / per * 8 + b % 8) * nvt + (b % per) / 8;
    }
    const int vt = b % nvt, unit = b / nvt;
    const int n = unit / H, h = unit % H;
    const int c0 = vt * BVs;
    for (int idx = tid; idx < DK * BVs; idx += NT) {
        const int c = idx / BVs, j = idx % BVs;
        const float x = s0 ? s0[(((int64_t)n * H + h) * DK + c) * Dv + c0 + j] : 0.f;
        sS[c][j] = x;
        if constexpr (DK == 128) {
            const __bf16 hi = (__bf16)x;
            sSh[j][c] = hi;
            sSl[j][c] = (__bf16)(x - (float)hi);
        }
    }
    __syncthreads();
    if constexpr (DK == 128) {
        // S_new = A S + B on the matrix cores: 8 row tiles of 16 x 16, one per
        // wave, each product as three bf16 products of hi and lo parts
        // (A_hi S_hi + A_hi S_lo + A_lo S_hi, float32 accumulation; the lo lo
        // term is below 2^-17 of the product). A and B go through two
        // register sets: step p stages its set
        // into LDS and the accumulators and then loads step p + 2's into it, so
        // every load has two steps to land (past the last step the loads repeat
        // it).
        const int lane = tid & 63, w = tid >> 6, l16 = lane & 15, lg = lane >> 4;
        struct Regs {
            float4 a[kPer];
            float b[4];
        };
        auto issue = [&](int p, Regs& R) {
            const int64_t seg = (int64_t)n * P + (p < P ? p : P - 1);
            const float4* a4 = reinterpret_cast<const float4*>(A + (seg * H + h) * (int64_t)DK * DK);
            const float* b = Bst + (seg * H + h) * (int64_t)DK * Dv;
#pragma unroll
            for (int u = 0; u < kPer; ++u) R.a[u] = a4[tid + NT * u];
#pragma unroll
            for (int i = 0; i < 4; ++i) R.b[i] = b[(int64_t)(16 * w + 4 * lg + i) * Dv + c0 + l16];
        };
        // one step; false once the chain is done
        auto step = [&](int p, Regs& R) -> bool {
            const int64_t seg = (int64_t)n * P + p;
            float* sin = Sin + (seg * H + h) * (int64_t)DK * Dv;
            for (int idx = tid; idx < DK * BVs; idx += NT) {
                const int c = idx / BVs, j = idx % BVs;
                sin[(int64_t)c * Dv + c0 + j] = sS[c][j];
            }
            if (p == P - 1 && !sT) return false;
#pragma unroll
            for (int u = 0; u < kPer; ++u) {
                const int q = tid + NT * u;
                const int r = q / (DK / 4), c = (q % (DK / 4)) * 4;
                sA[r][c] = R.a[u].x; sA[r][c + 1] = R.a[u].y; sA[r][c + 2] = R.a[u].z; sA[r][c + 3] = R.a[u].w;
            }
            f32x4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = R.b[i];
            __syncthreads();
            issue(p + 2, R);
            // from a zero initial state, S_in(1) = B(0): A(0) is not read (the
            // bf16 split does not compute it)
            if (p > 0 || s0) {
                // every operand is read from LDS before the products start (one
                // LDS round trip per product would set the pace); lane (l16, lg)
                // of k-block kb holds A[16w + l16][32kb + 8lg + s] and
                // S[32kb + 8lg + s][l16], s = 0..7, and the three parts
                // accumulate in separate chains
                constexpr int KB = DK / 32;
                bf16x8 ah[KB], al[KB], bh[KB], bl[KB];
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const float4 x0 = *reinterpret_cast<const float4*>(&sA[16 * w + l16][32 * kb + 8 * lg]);
                    const float4 x1 = *reinterpret_cast<const float4*>(&sA[16 * w + l16][32 * kb + 8 * lg + 4]);
                    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const __bf16 hi = (__bf16)xs[e];
                        ah[kb][e] = hi;
                        al[kb][e] = (__bf16)(xs[e] - (float)hi);
                    }
                    bh[kb] = *reinterpret_cast<const bf16x8*>(&sSh[l16][32 * kb + 8 * lg]);
                    bl[kb] = *reinterpret_cast<const bf16x8*>(&sSl[l16][32 * kb + 8 * lg]);
                }
                f32x4 phh = acc, phl = {0.f, 0.f, 0.f, 0.f}, plh = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    phh = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[kb], bh[kb], phh, 0, 0, 0);
                    phl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[kb], bl[kb], phl, 0, 0, 0);
                    plh = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[kb], bh[kb], plh, 0, 0, 0);
                }
                acc = phh + (phl + plh);
            }
            __syncthreads();
            bf16x4 hi4, lo4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sS[16 * w + 4 * lg + i][l16] = acc[i];
                const __bf16 hb = (__bf16)acc[i];   // (through a scalar)
                hi4[i] = hb;
                lo4[i] = (__bf16)(acc[i] - (float)hb);
            }
            *reinterpret_cast<bf16x4*>(&sSh[l16][16 * w + 4 * lg]) = hi4;
            *reinterpret_cast<bf16x4*>(&sSl[l16][16 * w + 4 * lg]) = lo4;
            __syncthreads();
            return p + 1 < P;
        };
        Regs R0, R1;
        issue(0, R0);
        issue(1, R1);
        for (int p = 0;; p += 2) {
            if (!step(p, R0)) break;
            if (!step(p + 1, R1)) break;
        }
    } else {
        for (int p = 0; p < P; ++p) {
            const int64_t seg = (int64_t)n * P + p;
            float* sin = Sin + (seg * H + h) * (int64_t)DK * Dv;
            for (int idx = tid; idx < DK * BVs; idx += NT) {
                const int c = idx / BVs, j = idx % BVs;
                sin[(int64_t)c * Dv + c0 + j] = sS[c][j];
            }
            if (p == P - 1 && !sT) break;
            // S <- A(p) S + B(p)
            const float4* a4 = reinterpret_cast<const float4*>(A + (seg * H + h) * (int64_t)DK * DK);
            const float* b = Bst + (seg * H + h) * (int64_t)DK * Dv;
            float4 ra[kPer];
    #pragma unroll
            for (int u = 0; u < kPer; ++u) {
                const int q = tid + NT * u;
                ra[u] = q < kQuads ? a4[q] : float4{0.f, 0.f, 0.f, 0.f};
            }
            float rb[kOut];
    #pragma unroll
            for (int u = 0; u < kOut; ++u) {
                const int idx = tid + NT * u;
                rb[u] = idx < DK * BVs ? b[(int64_t)(idx / BVs) * Dv + c0 + idx % BVs] : 0.f;
            }
    #pragma unroll
            for (int u = 0; u < kPer; ++u) {
                const int q = tid + NT * u;
                if (q < kQuads) {
                    const int r = q / (DK / 4), c = (q % (DK / 4)) * 4;
                    sA[r][c] = ra[u].x; sA[r][c + 1] = ra[u].y; sA[r][c + 2] = ra[u].z; sA[r][c + 3] = ra[u].w;
                }
            }
            __syncthreads();
            {
                float out[kOut];
    #pragma unroll
                for (int u = 0; u < kOut; ++u) {
                    const int idx = tid + NT * u;
                    const int c = idx / BVs, j = idx % BVs;
                    float acc = rb[u];
                    if (idx < DK * BVs) {
    #pragma unroll 8
                        for (int i = 0; i < DK; ++i) acc += sA[c][i] * sS[i][j];
                    }
                    out[u] = acc;
                }
                __syncthreads();
    #pragma unroll
                for (int u = 0; u < kOut; ++u) {
                    const int idx = tid + NT * u;
                    if (idx < DK * BVs) sS[idx / BVs][idx % BVs] = out[u];
                }
            }
            __syncthreads();
        }
    }
    if (sT) {
        for (int idx = tid; idx < DK * BVs; idx += NT) {
            const int c = idx / BVs, j = idx % BVs;
            sT[(((int64_t)n * H + h) * DK + c) * Dv + c0 + j] = sS[c][j];
        }
    }
}

// The output pass of the bf16 d=128 split. Over segment p the state at row t
// is S_t = A_t S_in(p) + B_t (A_t, B_t: the maps of the segment's rows up to
// t), so its output is o_t = o_B(t) + S_in(p)ᵀ oA(t), where o_B is the output
// from a zero entry state and oA(t) = scale A_tᵀ q_t the output of the A pass
// (v = 0 from the identity, Dk columns). o holds o_B for every segment (exact
// already in a sequence's first segment); this adds the second term to the
// rows of segments p >= 1 and rounds once more to bf16.
//
// One workgroup of four waves per (segment, head, slice r of R): the 64-row
// blocks r, r + R, ... of the segment; wave w takes output columns
// 32w..32w+31 (two 16-column tiles). The products run on the matrix cores as
// D = S_inᵀ oAᵀ (16x16x32 bf16): S_in split into bf16 hi + lo parts (float32
// accuracy for the state) held in registers, oA exact (it is stored in bf16).
// Tile t's operand row a stands for output column 8(a/4) + 4t + a%4 of the
// wave's 32, so that lane group lg ends up with the 8 consecutive columns
// 8lg..8lg+7 of its row from the two tiles, and o is read and written in
// 16-byte pieces, 64 contiguous bytes per row and instruction (8-byte pieces,
// 32 bytes per row, cost 42 of the kernel's 68 us at 12 heads x 32768).
// A block's oA rows (16 KB) go straight from global memory to LDS, once for
// the four waves, in a ring of three buffers: blocks b+1 and b+2 (and their o
// rows, into registers) are in flight while block b is computed, and the wait
// before block b counts only its own loads, not the stores of the blocks
// before it. In LDS, 16-byte piece c of row i sits
// at position c ^ (i % 16) of the row, so the 16 rows that one operand read
// touches fall in different banks.
constexpr int kCorrBlockBytes = 64 * 256;
// s_waitcnt operand that waits until at most n vector-memory operations are
// outstanding (gfx9 encoding: vmcnt bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their maxima)
constexpr int vmcnt_wait(int n) { return ((n >> 4) << 14) | 0x0F70 | (n & 15); }
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
// The workgroup barrier of the correction loop, with no memory fence. A fence
// (that of __syncthreads(), or one on LDS alone) waits for every global access
// of the wave, the global-to-LDS loads of later blocks included. Here each
// wave has waited, with an exact count, for its own loads of the block it is
// about to read, and has consumed its reads of the buffer that the next loads
// overwrite, so the barrier only has to align the waves; the empty asm keeps
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
// A buffer descriptor over [base, base + bytes), built from wave-uniform
// values (the stores through it then need no per-lane loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, int64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const int n = __builtin_amdgcn_readfirstlane((int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), 0, n, 0x00020000);
}
__global__ __launch_bounds__(256, 2) void split_correct_kernel(const int32_t* cu, int32_t T0, int32_t P, int32_t H,
                                                               int32_t R, const float* Sin, const __bf16* oA,
                                                               __bf16* o) {
    __shared__ __attribute__((aligned(16))) char buf[3][kCorrBlockBytes];
    const int r = blockIdx.x % R;
    const int unit = blockIdx.x / R;
    const int seg = unit / H, h = unit % H;
    if (seg % P == 0) return;                       // the whole workgroup
    int64_t bos, len;
    split_segment(cu, T0, P, 2, seg, bos, len);
    const int64_t eos = bos + len;
    if ((int64_t)r * 64 >= eos - bos) return;       // the whole workgroup
    const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index (uniform)
    const int64_t rstride = (int64_t)H * 128;       // elements between consecutive rows of oA and o
    // Issue block r0's loads: its oA rows into LDS buffer `bi` (wave w: rows
    // 16w..16w+15, four rows per instruction; rows past the segment end read
    // its last row) and this wave's o rows (row li of tile rt, columns
    // 32w + 8lg..+7) into ob.
    auto issue = [&](int64_t r0, int bi, uint4 (&ob)[4]) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = 16 * w + 4 * k + (lane >> 4);                  // row in the block
            const int64_t row = r0 + i < eos ? r0 + i : eos - 1;
            const int c = (lane & 15) ^ (i & 15);                          // piece this lane stores
            __builtin_amdgcn_global_load_lds(
                (const void*)(oA + row * rstride + (int64_t)h * 128 + 8 * c),
                (__attribute__((address_space(3))) void*)(buf[bi] + (16 * w + 4 * k) * 256), 16, 0, 0);
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const int64_t row = r0 + 16 * rt + li < eos ? r0 + 16 * rt + li : eos - 1;
            ob[rt] = *reinterpret_cast<const uint4*>(o + row * rstride + (int64_t)h * 128 + 32 * w + 8 * lg);
        }
    };
    // A operands: lane (li, lg) of column tile t, k-step ks holds
    // S_in[32ks + 8lg + j][32w + 8(li/4) + 4t + li%4], j = 0..7
    const float* S = Sin + ((int64_t)seg * H + h) * 128 * 128;
    bf16x8 shi[2][4], slo[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int col = 32 * w + 8 * (li >> 2) + 4 * t + (li & 3);
                const float x = S[(int64_t)(32 * ks + 8 * lg + j) * 128 + col];
                const __bf16 hi = (__bf16)x;
                shi[t][ks][j] = hi;
                slo[t][ks][j] = (__bf16)(x - (float)hi);
            }
    uint4 ob0[4], ob1[4], ob2[4];
    auto compute = [&](int64_t r0, int bi, const uint4 (&ob)[4]) {
        // o from row r0 to the block's end or the segment's, whichever comes first
        const int64_t nrows = eos - r0 < 64 ? eos - r0 : 64;
        const __amdgpu_buffer_rsrc_t ro = uniform_rsrc(o + r0 * rstride, nrows * rstride * 2);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            // B operand: row 16rt + li, channels 32ks + 8lg..+7 (piece 4ks + lg)
            const int i = 16 * rt + li;
            f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 b = *reinterpret_cast<const bf16x8*>(buf[bi] + i * 256 + 16 * ((4 * ks + lg) ^ li));
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(shi[t][ks], b, acc[t], 0, 0, 0);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(slo[t][ks], b, acc[t], 0, 0, 0);
                }
            }
            // D: lane (li, lg) holds row li of the tile, columns 32w + 8lg + 4t + i;
            // every store is issued, and those of rows past the segment end fall
            // outside the descriptor's range, where the hardware drops them
            const uint32_t in[4] = {ob[rt].x, ob[rt].y, ob[rt].z, ob[rt].w};
            uint32_t out[4];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const float y0 = __uint_as_float(in[2 * t] << 16) + acc[t][0];
                const float y1 = __uint_as_float(in[2 * t] & 0xffff0000u) + acc[t][1];
                const float y2 = __uint_as_float(in[2 * t + 1] << 16) + acc[t][2];
                const float y3 = __uint_as_float(in[2 * t + 1] & 0xffff0000u) + acc[t][3];
                out[2 * t] = pack2_bf16(y0, y1);
                out[2 * t + 1] = pack2_bf16(y2, y3);
            }
            const int off = 2 * (i * (int)rstride + 128 * h + 32 * w + 8 * lg);
            __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{out[0], out[1], out[2], out[3]}, ro, off, 0, 0);
        }
    };
    // Every block issues the same vector-memory operations per wave, past the
    // segment end too (its loads then repeat the last row): issue() makes 8
    // loads (4 into LDS, 4 into registers), compute() 4 stores. Before block k
    // the operations issued after its loads are block k+1's loads (block 0),
    // then block k-1's stores and block k+2's loads (block 1), then block k-2's
    // stores as well, so the wait leaves 8, 12 or 16 outstanding, and the
    // compiler, which sees the same operations on every path, needs no wait of
    // its own.
    constexpr int kLoads = 8, kStores = 4;
    using Wait0 = std::integral_constant<int, kLoads>;
    using Wait1 = std::integral_constant<int, kLoads + kStores>;
    using Wait2 = std::integral_constant<int, kLoads + 2 * kStores>;
    // every wave runs the same block sequence, so the barriers match
    const int64_t step = (int64_t)R * 64;
    int64_t rk = bos + (int64_t)r * 64;
    issue(rk, 0, ob0);
    issue(rk + step, 1, ob1);
    // one block: its loads landed for every wave, the buffer of block k-1 is
    // free for block k+2. Blocks 0 and 1 run before the loop, so that every
    // stage in it waits with the same count: with the count chosen at run
    // time the compiler lost track of the register loads and waited for all
    // of them before the first use in one stage of three.
    auto stage = [&](auto wait_n, int bi, const uint4 (&ob)[4], int bn, uint4 (&obn)[4]) -> bool {
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(decltype(wait_n)::value));
        lds_barrier();
        issue(rk + 2 * step, bn, obn);
        compute(rk, bi, ob);
        if (rk + step >= eos) return false;
        rk += step;
        return true;
    };
    if (stage(Wait0{}, 0, ob0, 2, ob2) && stage(Wait1{}, 1, ob1, 0, ob0)) {
        for (;;) {
            if (!stage(Wait2{}, 2, ob2, 1, ob1)) break;
            if (!stage(Wait2{}, 0, ob0, 2, ob2)) break;
            if (!stage(Wait2{}, 1, ob1, 0, ob0)) break;
        }
    }
    // the loads issued past the end still write LDS: they land before the
    // workgroup ends and its LDS goes to another
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
}

unsigned grid_for(int64_t n) {
    const int64_t b = (n + 255) / 256;
    return (unsigned)(b < 8192 ? (b > 0 ? b : 1) : 8192);
}

hipError_t chunk_forward(const ChunkArgs& a, hipStream_t s) {
    return chunk_mfma_supported(a) ? launch_chunk_mfma(a, s) : launch_chunk_generic(a, s);
}

}  // namespace

SplitLayout split_layout(const ChunkArgs& a, int32_t P) {
    SplitLayout L;
    const int64_t segs = (int64_t)a.N * P;
    auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
    int64_t off = 0;
    L.seg_cu = off;  off += up((segs + 1) * 4);
    L.ident = off;   off += up(segs * a.H * (int64_t)a.Dk * a.Dk * 4);          // identity entry states, then A
    L.Bst = off;     off += up(segs * a.H * (int64_t)a.Dk * a.Dv * 4);
    L.Sin = off;     off += up(segs * a.H * (int64_t)a.Dk * a.Dv * 4);
    L.oA = off;
    if (chunk_mfma_supported(a)) off += up((int64_t)a.B * a.T * a.H * a.Dk * 2);   // the A pass's outputs
    L.bytes = off;
    return L;
}

hipError_t launch_chunk_fwd_split(const ChunkArgs& a, int32_t P, void* workspace, hipStream_t s) {
    const SplitLayout L = split_layout(a, P);
    char* ws = static_cast<char*>(workspace);
    int32_t* seg_cu = reinterpret_cast<int32_t*>(ws + L.seg_cu);
    float* AI = reinterpret_cast<float*>(ws + L.ident);
    float* Bst = reinterpret_cast<float*>(ws + L.Bst);
    float* Sin = reinterpret_cast<float*>(ws + L.Sin);
    const int64_t segs = (int64_t)a.N * P;
    hipError_t e;


    // the packed view of the input: one row of B*T tokens, N*P sequences
    ChunkArgs seg = a;
    seg.B = 1;
    seg.T = a.B * a.T;
    seg.N = (int32_t)segs;
    seg.cu = seg_cu;
    // 1. B (no outputs written)
    ChunkArgs p1 = seg;
    p1.s0 = nullptr;
    p1.sT = Bst;
    p1.o = nullptr;
    if (chunk_mfma_supported(p1)) {
        // bf16, d = 128: the A and B passes in one launch, the column blocks of A
        // beside those of B on the same XCD (q, k, g and beta come from HBM once
        // for both). B writes o (exact in first segments, which start from the
        // initial state, so their B is already S_in(1)); A writes A_tᵀ q_t. The
        // scan from a zero state then gives S_in(p), and the output pass adds
        // S_in(p)ᵀ A_tᵀ q_t to the other segments' rows.
        __bf16* oA = reinterpret_cast<__bf16*>(ws + L.oA);
        p1.cu = a.cu;     // the segments' bounds are computed in the kernels (split_segment)
        p1.o = a.o;
        p1.aug = true;
        p1.aug_T = a.T;
        p1.aug_P = P;
        p1.aug_s0_first = a.s0;
        p1.aug_sT = AI;
        p1.aug_o = oA;
        if ((e = launch_chunk_mfma(p1, s)) != hipSuccess) return e;
        split_scan_kernel<128><<<dim3((unsigned)(a.N * a.H * (a.Dv / 16))), dim3(scan_threads<128>()), 0, s>>>(
            AI, Bst, nullptr, Sin, a.sT, a.N, a.H, a.Dv, P);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (!a.o) return hipSuccess;
        const int64_t units = segs * a.H;
        // a grid resident at once (2 workgroups per CU at this kernel's registers)
        const int R = (int)std::max<int64_t>(1, std::min<int64_t>(16, 512 / units));
        split_correct_kernel<<<dim3((unsigned)(units * R)), dim3(256), 0, s>>>(a.cu, a.T, P, a.H, R, Sin, oA,
                                                                               static_cast<__bf16*>(a.o));
        return hipGetLastError();
    } else {
        split_offsets_kernel<<<dim3((unsigned)((a.N + 255) / 256)), dim3(256), 0, s>>>(a.cu, a.N, a.T, P, seg_cu);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        fill_identity_kernel<<<dim3(grid_for(segs * a.H * a.Dk * a.Dk)), dim3(256), 0, s>>>(AI, segs * a.H, a.Dk);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = chunk_forward(p1, s)) != hipSuccess) return e;
        // 2. A: identity entry states, v = 0 (read from an empty range), d_v = d_k, no outputs
        ChunkArgs p2 = seg;
        p2.v = nullptr;
        p2.Dv = a.Dk;
        p2.s0 = AI;
        p2.sT = AI;   // each state tile is read before it is written
        p2.o = nullptr;
        if ((e = chunk_forward(p2, s)) != hipSuccess) return e;
    }
    // 3. entry states of every segment, and the final states
    switch (a.Dk) {
        case 16: split_scan_kernel<16><<<dim3((unsigned)(a.N * a.H * (a.Dv / 16))), dim3(256), 0, s>>>(
                     AI, Bst, a.s0, Sin, a.sT, a.N, a.H, a.Dv, P); break;
        case 32: split_scan_kernel<32><<<dim3((unsigned)(a.N * a.H * (a.Dv / 16))), dim3(256), 0, s>>>(
                     AI, Bst, a.s0, Sin, a.sT, a.N, a.H, a.Dv, P); break;
        case 64: split_scan_kernel<64><<<dim3((unsigned)(a.N * a.H * (a.Dv / 16))), dim3(256), 0, s>>>(
                     AI, Bst, a.s0, Sin, a.sT, a.N, a.H, a.Dv, P); break;
        default: split_scan_kernel<128><<<dim3((unsigned)(a.N * a.H * (a.Dv / 16))), dim3(scan_threads<128>()), 0, s>>>(
                     AI, Bst, a.s0, Sin, a.sT, a.N, a.H, a.Dv, P); break;
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // 4. the outputs, every segment from its entry state
    ChunkArgs p4 = seg;
    p4.s0 = Sin;
    p4.sT = nullptr;
    return chunk_forward(p4, s);
}

// Static scratch for the split entry point that allocates nothing
// (kda_chunk_fwd_split_static): the split's workspace (segment offsets, the
// identity / A states, the B states and the entry states) lives in this
// file-scope array, of which every device holds its own copy from module load
// to the end of the process. In host code the array's name is only a
// host-side stand-in, so its device address is looked up once per device with
// hipGetSymbolAddress and only that address is ever passed to a kernel. Every
// call on one device shares the array; calls that overlap in time on one
// device (other streams, other threads) race on it.
static __device__ __align__(256) char scratch[kSplitStaticScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

void* split_static_scratch() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace kda
