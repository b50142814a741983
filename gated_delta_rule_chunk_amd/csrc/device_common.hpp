// Small device helpers shared by the KDA kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// exp(x) on the hardware base-2 exponential; |x| stays below ~350 on every
// path that uses it, so the only loss is the rounding of x*log2(e).
__device__ __forceinline__ float fast_exp(float x) {
    return __builtin_amdgcn_exp2f(x * kLog2e);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t lo16) {
    return __uint_as_float(lo16 << 16);
}

// Unpack 8 bf16 values held in a 16-byte word.
__device__ __forceinline__ void unpack8(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x << 16);
    f[1] = __uint_as_float(u.x & 0xffff0000u);
    f[2] = __uint_as_float(u.y << 16);
    f[3] = __uint_as_float(u.y & 0xffff0000u);
    f[4] = __uint_as_float(u.z << 16);
    f[5] = __uint_as_float(u.z & 0xffff0000u);
    f[6] = __uint_as_float(u.w << 16);
    f[7] = __uint_as_float(u.w & 0xffff0000u);
}

// Round-to-nearest-even float -> bf16 bit pattern.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}

// Two floats -> packed bf16 pair (a in the low half). Written as a vector
// construction so it compiles to a single v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
    const bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// The intra-sequence split's cut: sequence m / P (offsets cu, or rows of T0
// tokens when cu is null) of length L is cut into P segments, the first of
// w0 shares and the others of one share each, a share being
// roundup(ceil(L / (P - 1 + w0)), 64) rows; the last segments are shorter or
// empty. Returns segment m's first token and length. (Where the first segment
// runs half the passes of the others, w0 = 2 gives every segment the same
// work.)
constexpr int kSplitSegAlign = 64;
__device__ __forceinline__ void split_segment(const int32_t* cu, int32_t T0, int32_t P, int32_t w0, int64_t m,
                                              int64_t& bos, int64_t& len) {
    const int64_t sq = m / P, p = m % P;
    const int64_t b0 = cu ? cu[sq] : sq * T0;
    const int64_t L = cu ? (int64_t)cu[sq + 1] - cu[sq] : T0;
    const int64_t shares = P - 1 + w0;
    int64_t seg = (L + shares - 1) / shares;
    seg = (seg + kSplitSegAlign - 1) / kSplitSegAlign * kSplitSegAlign;
    const int64_t s0 = p == 0 ? 0 : (w0 + p - 1) * seg, s1 = (w0 + p) * seg;
    const int64_t start = s0 < L ? s0 : L;
    const int64_t end = s1 < L ? s1 : L;
    bos = b0 + start;
    len = end - start;
}

// Load element i of an input that is either float or bf16.
template <typename T> __device__ __forceinline__ float load_elem(const T* p, int64_t i);
template <> __device__ __forceinline__ float load_elem<float>(const float* p, int64_t i) {
    return p[i];
}
template <> __device__ __forceinline__ float load_elem<__bf16>(const __bf16* p, int64_t i) {
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
}

template <typename T> __device__ __forceinline__ void store_elem(T* p, int64_t i, float v);
template <> __device__ __forceinline__ void store_elem<float>(float* p, int64_t i, float v) {
    p[i] = v;
}
template <> __device__ __forceinline__ void store_elem<__bf16>(__bf16* p, int64_t i, float v) {
    reinterpret_cast<uint16_t*>(p)[i] = f32_to_bf16_bits(v);
}

}  // namespace kda
