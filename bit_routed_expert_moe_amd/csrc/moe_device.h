// moe_device.h -- device-side building blocks for the gfx950 MoE kernels.
//
// Dequantised dot products.  A packed dword w holds 8 consecutive 4-bit
// weights q0..q7 (q_j in bits [4j, 4j+4)).  Four fp16 pairs are formed with
// one and-or each (plus one shared shift) by placing a nibble inside the
// mantissa of the fp16 value 1024 (bits 0x6400):
//     P0 = (w      & 0x000F000F) | 0x64006400  -> (1024 + q0,    1024 + q4)
//     P1 = (w      & 0x00F000F0) | 0x64006400  -> (1024 + 16 q1, 1024 + 16 q5)
//     P2 = (w >> 8 & 0x000F000F) | 0x64006400  -> (1024 + q2,    1024 + q6)
//     P3 = (w >> 8 & 0x00F000F0) | 0x64006400  -> (1024 + 16 q3, 1024 + 16 q7)
// and fed to v_dot2_f32_f16 against activation pairs prepared to match:
//     X0 = (a0, a4), X1 = (a1/16, a5/16), X2 = (a2, a6), X3 = (a3/16, a7/16)
// (a = activations times a per-vector power of two).  Every product of two
// fp16 values is exact in fp32 and
//     sum_pairs dot2(P, X) = sum_i q_i a_i + 1024 * sum_i a'_i
// where a'_i is the fp16 value actually used (a_i or a_i/16).  The second term,
// K = 1024 * sum a', is computed once per 64-group (in double) and subtracted.
// The affine group then contributes  scale * (acc - K) / 2^e + bias * sum(x).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                  c, false);
}

// The fp16 pair (1024, 1024) in a register the compiler cannot fold: with the
// constant hidden, (w & mask) | M selects one v_and_or_b32 (mask in an SGPR)
// instead of a v_and_b32 and a v_or_b32 with literal operands.
__device__ __forceinline__ uint32_t magic_1024x2() {
    uint32_t m = 0x64006400u;
    asm("" : "+v"(m));
    return m;
}

// acc0 gathers the q0/q4/q2/q6 pairs, acc1 the x16 pairs; x points at 4 dwords.
__device__ __forceinline__ void dot_nib8(uint32_t w, const uint32_t* x, float& acc0, float& acc1) {
    const uint32_t M = magic_1024x2();
    const uint32_t w8 = w >> 8;
    acc0 = dot2((w & 0x000F000Fu) | M, x[0], acc0);
    acc1 = dot2((w & 0x00F000F0u) | M, x[1], acc1);
    acc0 = dot2((w8 & 0x000F000Fu) | M, x[2], acc0);
    acc1 = dot2((w8 & 0x00F000F0u) | M, x[3], acc1);
}

// 2-bit codes: a dword w holds 16 codes, input i in bits [2i, 2i+2); pair j
// is (q_j, q_{8+j}), j = 0..7, the halves' fields at bits 2j and 16+2j.  Left
// in place, field j or-ed with 0x6400 is the fp16 1024 + 4^j q for j < 5 (it
// stays within the 10 mantissa bits); fields 5..7 are taken the same way from
// w >> 10, as 1024 + 4^(j-5) q.  The activation dwords x[j] = (a_j, a_{8+j})
// carry the inverse power (crumb_scale_log2).  acc0 gathers the even j, acc1
// the odd j.  One and-or per pair plus one shift per dword.
__device__ __forceinline__ void dot_crumb16(uint32_t w, const uint32_t* x, float& acc0, float& acc1) {
    const uint32_t M = magic_1024x2();
    const uint32_t v = w >> 10;
    acc0 = dot2((w & 0x00030003u) | M, x[0], acc0);
    acc1 = dot2((w & 0x000C000Cu) | M, x[1], acc1);
    acc0 = dot2((w & 0x00300030u) | M, x[2], acc0);
    acc1 = dot2((w & 0x00C000C0u) | M, x[3], acc1);
    acc0 = dot2((w & 0x03000300u) | M, x[4], acc0);
    acc1 = dot2((v & 0x00030003u) | M, x[5], acc1);
    acc0 = dot2((v & 0x000C000Cu) | M, x[6], acc0);
    acc1 = dot2((v & 0x00300030u) | M, x[7], acc1);
}

// log2 of the factor that pair j of dot_crumb16 needs on its activations
__device__ __forceinline__ int crumb_scale_log2(int j) { return j < 5 ? -2 * j : -2 * (j - 5); }

__device__ __forceinline__ float f16lo(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
}
__device__ __forceinline__ float f16hi(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}
__device__ __forceinline__ uint16_t f16bits(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);  // round to nearest even
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float v) {  // round to nearest even, finite v
    uint32_t u = __builtin_bit_cast(uint32_t, v);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Power-of-two exponent e such that max_abs * 2^e < 2^14 (0 when max_abs is 0).
__device__ __forceinline__ int act_exponent(float max_abs) {
    if (!(max_abs > 0.0f)) return 0;
    int p;
    frexpf(max_abs, &p);  // max_abs = m * 2^p, m in [0.5, 1)
    int e = 14 - p;
    return e < -120 ? -120 : (e > 120 ? 120 : e);
}

// ---- wave64 reductions (DPP within rows of 16, then across the 4 rows) ----
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over all 64 lanes; every lane gets the same value, the order is fixed.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp<0x124>(v);  // row_ror:4
    v += dpp<0x128>(v);  // row_ror:8
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (r0 + r1) + (r2 + r3);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int lane) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

// Max over all 64 lanes (DPP within rows, then the 4 row results); every lane
// gets the same value.
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x124>(v));
    v = fmaxf(v, dpp<0x128>(v));
    const int iv = __builtin_bit_cast(int, v);
    return fmaxf(fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 0)),
                       __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 16))),
                 fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 32)),
                       __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 48))));
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint64_t lo = dpp_u32<CTRL>((uint32_t)u), hi = dpp_u32<CTRL>((uint32_t)(u >> 32));
    return __builtin_bit_cast(double, lo | (hi << 32));
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint64_t lo = readlane_u32((uint32_t)u, lane), hi = readlane_u32((uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(double, lo | (hi << 32));
}

// Sum over all 64 lanes in double, fixed order; every lane gets the same value.
__device__ __forceinline__ double wave_sum_d(double v) {
    v += dpp_f64<0xB1>(v);
    v += dpp_f64<0x4E>(v);
    v += dpp_f64<0x124>(v);
    v += dpp_f64<0x128>(v);
    return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

template <typename T>
__device__ __forceinline__ T ldg_nt(const T* p) { return __builtin_nontemporal_load(p); }

}  // namespace moe
