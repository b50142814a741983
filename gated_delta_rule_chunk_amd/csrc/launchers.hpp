// Internal launch interface between the C ABI (kda_api.hip) and the kernels.
// Arguments are validated by the caller; these functions only launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct ChunkArgs {
    const void* q;
    const void* k;
    const void* v;            // nullptr: v = 0 (internal passes of the split)
    const void* g;
    const void* beta;
    const float* s0;          // [N,H,Dk,Dv] or nullptr
    const int32_t* cu;        // [N+1] or nullptr
    void* o;                  // nullptr: outputs not written (internal passes of the split)
    float* sT;                // [N,H,Dk,Dv] or nullptr
    int32_t B, T, H, Dk, Dv, N, chunk;
    int32_t chunk_req = 0;    // chunk_size as the caller passed it (0 = the kernel's own)
    float scale;
    bool bf16;
    // gate, beta and normalisation prologue: when set, q and k hold the raw
    // projections (normalised in the kernel), g the gate logits and beta the
    // beta logits
    bool prologue = false;
    const float* A_log = nullptr;     // [Dk]
    const float* dt_bias = nullptr;   // [H*Dk]
    float gate_lb = 0.f;
    float l2_eps = 0.f;
    // bounded waits between waves: polls before giving up, and the device
    // word that counts give-ups (set by the C ABI for every launch)
    int spin_limit = 1 << 22;
    unsigned int* status = nullptr;
    // short convolution of v fused in (kda_chunk_fwd_conv; bf16, Dk = Dv = 128,
    // with the prologue): v is the raw projection
    bool conv = false;
    const float* conv_wv = nullptr;  // taps of v: [H*Dv][4]
    const float* conv_sv = nullptr;  // conv state of v: [N][3][H*Dv], or null (zeros)
    bool conv_act = false;           // SiLU after the convolution
    // the split's A and B passes in one launch (bf16, Dk = Dv = 128): the
    // sequences are the segments, aug_P per original sequence (bounds by
    // split_segment, first-segment weight 2, from the original cu and aug_T;
    // N counts segments), and every
    // (segment, head) gets twice the column blocks. The first set runs with v
    // from a zero entry state (aug_s0_first of the sequence in its first
    // segment) into sT and o (B); the second, skipped in first segments, with
    // v = 0 from the identity into aug_sT and aug_o (A).
    bool aug = false;
    int32_t aug_P = 1;
    int32_t aug_T = 0;                     // T of the original call (its cu in cu, or null)
    const float* aug_s0_first = nullptr;   // [N / aug_P, H, Dk, Dv] or nullptr
    float* aug_sT = nullptr;
    void* aug_o = nullptr;                 // like o, with Dk columns
};

// The device status word of the current device and the poll limit of every
// bounded wait (both owned by the C ABI).
unsigned int* device_status_word();
int wait_spin_limit();

struct StepArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* beta;
    float* cache;              // [n_slots][H][Dk][Dv]
    const int32_t* slots;      // [Nb] or nullptr (row r -> slot r)
    void* o;
    int32_t n_slots;           // rows whose slot lies outside [0, n_slots) are padding
    int32_t Nb, H, Dk, Dv;
    float scale;
    bool bf16;
    // decode from raw projections: q and k hold the raw projections
    // (normalised in the kernel), g the gate logits and beta the beta logits
    bool prologue = false;
    const float* A_log = nullptr;     // [Dk]
    const float* dt_bias = nullptr;   // [H*Dk]
    float gate_lb = 0.f;
    float l2_eps = 0.f;
    // with the prologue, the short-convolution step of q, k and v before it:
    // q, k and v hold the convolution inputs; per projection j (q, k, v) taps
    // [H*D][4] and a cache [n_slots][3][H*D] (D = Dk for q and k, Dv for v)
    // indexed by the row's slot and shifted in place
    bool conv = false;
    bool conv_act = false;            // SiLU after the convolution
    const float* conv_w[3] = {nullptr, nullptr, nullptr};
    float* conv_cache[3] = {nullptr, nullptr, nullptr};
};

// Each returns hipSuccess or the launch error; they never synchronise.
struct ConvArgs {
    const void* x;             // [B,T,C]
    const float* w;            // [C][4]
    const float* state_in;     // [N][3][C] or nullptr
    const int32_t* cu;         // [N+1] or nullptr
    void* y;                   // [B,T,C]
    float* state_out;          // [N][3][C] or nullptr
    int32_t B, T, C, N;
    bool act, bf16;
};

struct ConvStepArgs {
    const void* x;             // [Nb][C]
    const float* w;            // [C][4]
    float* cache;              // [n_slots][3][C]
    const int32_t* slots;      // [Nb] or nullptr
    void* y;                   // [Nb][C]
    int32_t n_slots;           // rows whose slot lies outside [0, n_slots) are padding
    int32_t Nb, C;
    bool act, bf16;
};

// Backward of the chunk forward; gradients are float32.
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* beta;
    const void* d_o;           // [B,T,H,Dv], input dtype
    const float* s0;           // [N,H,Dk,Dv] or nullptr
    const int32_t* cu;         // [N+1] or nullptr
    const float* d_final;      // [N,H,Dk,Dv] or nullptr
    float* ws;                 // chunk entry states [slots][H][Dk][Dv]
    float* dq;                 // [B,T,H,Dk]
    float* dk;
    float* dv;                 // [B,T,H,Dv]
    float* dg;                 // [B,T,H,Dk]
    float* dbeta;              // [B,T,H]
    float* d_s0;               // [N,H,Dk,Dv] or nullptr
    int32_t B, T, H, Dk, Dv, N;
    float scale;
    bool bf16;
    bool g_ge_m5 = true;       // g >= -5 holds (the matrix-core kernel relies on it)
    bool x_bf16 = false;       // with bf16 false: v and d_o are bf16 (matrix-core path only)
    bool zero_grads = false;   // (set by the launcher) the T/P/KK kernel zeroes dq, dk, dg, dbeta
    // the device's status words (the matrix-core T/P/KK kernel counts log-decays
    // outside [-5, 0] in word 1), or nullptr
    unsigned int* status = nullptr;
};

// The backward's workspace: a float32 chunk-entry state [H][Dk][Dv] per
// 16-row chunk slot (sequence n's chunks start at slot cu[n]/16 + n when
// packed, n*ceil(T/16) otherwise), then per (slot, head) the chunk's T, P
// and KK (3 x 16 x 16 floats).
__host__ __device__ inline int64_t chunk_bwd_slots(int32_t B, int32_t T, int32_t N, bool packed) {
    return packed ? (int64_t)T / 16 + N : (int64_t)B * ((T + 15) / 16);
}
__host__ __device__ inline int64_t chunk_bwd_ws_floats(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv,
                                                       int32_t N, bool packed) {
    return chunk_bwd_slots(B, T, N, packed) * H * ((int64_t)Dk * Dv + 3 * 16 * 16);
}
hipError_t launch_chunk_bwd(const BwdArgs& a, hipStream_t s);
bool chunk_bwd_mfma_supported(const BwdArgs& a);   // Dk = 128, Dv in {64, 128}

// Backward from raw projections through the gate, beta and L2-norm prologue.
struct PrologueBwdArgs {
    const void* q_raw;
    const void* k_raw;
    const void* g_logit;
    const void* beta_logit;
    const void* v;
    const void* d_o;
    const float* A_log;        // [Dk]
    const float* dt_bias;      // [H*Dk]
    float gate_lb, l2_eps;
    float *qf, *kf, *gf, *bf, *vf, *dof;   // prologue outputs, float32 (workspace)
    bool widen_x;                          // write v and dO widened to vf, dof
    float *dq, *dk, *dg, *dbeta;           // gradient buffers, transformed in place
    float *part_b, *part_A;                // per (token block, head, channel) partial sums (workspace)
    float *d_A_log, *d_dt_bias;
    int32_t B, T, H, Dk, Dv;
    bool bf16;
};
// Byte offsets in its workspace (256-aligned): the recurrence backward's own
// workspace first, then the float32 prologue outputs and the partial sums.
struct PrologueBwdLayout {
    int64_t core, qf, kf, gf, bf, vf, dof, part_b, part_A, bytes;
};
PrologueBwdLayout prologue_bwd_layout(int32_t B, int32_t T, int32_t H, int32_t Dk, int32_t Dv, int32_t N,
                                      bool packed);
hipError_t launch_prologue_bwd(const PrologueBwdArgs& p, const BwdArgs& core, hipStream_t s);
// The prologue alone (kda_prologue): q_raw, k_raw, g_logit, beta_logit, A_log,
// dt_bias, gate_lb, l2_eps, B, T, H, Dk and bf16 set, and qf, kf, gf, bf
// pointing at outputs in the input dtype (widen_x false).
hipError_t launch_prologue(const PrologueBwdArgs& p, hipStream_t s);

// Workspace of the intra-sequence split (byte offsets, 256-aligned).
struct SplitLayout {
    int64_t seg_cu, ident, Bst, Sin, oA, bytes;
};
SplitLayout split_layout(const ChunkArgs& a, int32_t P);
hipError_t launch_chunk_fwd_split(const ChunkArgs& a, int32_t P, void* workspace, hipStream_t s);
// The split's static scratch (kda_chunk_fwd_split_static): its size, and its
// device address on the current device (nullptr if it cannot be looked up).
constexpr size_t kSplitStaticScratchBytes = (size_t)128 << 20;
void* split_static_scratch();

// Backward of the short convolution: fwd holds the forward's arguments (x, w,
// state_in, cu, sizes, activation, dtype); gradients are float32.
struct ConvBwdArgs {
    ConvArgs fwd;
    const float* dy;           // [B,T,C]
    const float* d_final;      // [N][3][C] or nullptr
    float* dx;                 // [B,T,C]
    float* dw;                 // [C][4]
    float* d_state;            // [N][3][C] or nullptr
    float* part;               // [token blocks][C][4] workspace
    int32_t B, T, C, N;
};
int64_t short_conv_bwd_blocks(int32_t B, int32_t T);
hipError_t launch_short_conv_bwd(const ConvBwdArgs& a, hipStream_t s);

hipError_t launch_short_conv(const ConvArgs& a, hipStream_t s);
// Several convolutions of one layer's projections in one launch of each
// kernel (same dtype, activation, B, T and N; C may differ): the convolution
// of every one whose y is set, then the final state of every one whose
// state_out is set.
constexpr int kMaxConvSet = 3;
hipError_t launch_short_conv_set(const ConvArgs* a, int count, hipStream_t s);
hipError_t launch_short_conv_step(const ConvStepArgs& a, hipStream_t s);

hipError_t launch_chunk_mfma(const ChunkArgs& a, hipStream_t s);     // bf16, Dk=Dv=128, 16-row chunks
hipError_t launch_chunk_generic(const ChunkArgs& a, hipStream_t s);  // any supported dims
hipError_t launch_recurrent_step(const StepArgs& a, hipStream_t s);

bool chunk_mfma_supported(const ChunkArgs& a);

}  // namespace kda
