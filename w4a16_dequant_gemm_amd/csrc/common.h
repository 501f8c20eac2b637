// Device-side building blocks shared by the W4A16 kernels (gfx950 / CDNA4, wave64).
//
// Code layout.  A 32-bit word of the packed weight row holds 8 consecutive input
// columns k0..k7, element k_t in bits 4t..4t+3.  The kernels never rebuild the natural
// order: a word is split into four 16-bit pairs (k0,k4) (k1,k5) (k2,k6) (k3,k7) with one
// AND/OR each (the "exponent-bias" trick: OR-ing a nibble into the mantissa of a
// 16-bit float whose exponent makes one ulp equal to 1 yields bias + code exactly).
// Activations are permuted the same way once, when they are loaded, so every
// dot product sees matching pairs: per 8-column block the activation order is
// x0 x4 x1 x5 x2 x6 x3 x7.
//
// Dequantization x_hat = s * (u - z) (page "推理优化中“用精度换性能“的核心技术：量化",
// section 2.3; page "量化实战深入（GPTQ / AWQ / SmoothQuant / KV 量化）", section 二) is
// applied in two parts: the integer part (u - z) enters the dot products / MFMAs, the
// per-group scale s multiplies the fp32 partial sum of the group afterwards, so no
// rounded fp16/bf16 weight is ever formed.
//   fp16 activations: the pair holds the exact small integers (u - z); the bias 1024 and
//     the zero point are removed with one packed fp16 add (or fma), which is exact for
//     |z| <= 1024.
//   bf16 activations: gfx950 has no packed bf16 add, so the pair holds 128 + u (exact in
//     bf16); the MFMA/dot result is sum x*(128+u) and the group epilogue subtracts
//     (128 + z) * sum(x) in fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { DT_F16 = 0, DT_BF16 = 1 };

// fp16 bits -> float (exact).
__device__ __forceinline__ float h2f(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}
// bf16 bits -> float (exact).
__device__ __forceinline__ float bf2f(uint32_t b16) {
    return __builtin_bit_cast(float, b16 << 16);
}
// float -> fp16 / bf16 bits, round-to-nearest-even.
__device__ __forceinline__ uint16_t f2h_bits(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}
__device__ __forceinline__ uint16_t f2bf_bits(float v) {
    return __builtin_bit_cast(uint16_t, (__bf16)v);
}
template <int DT>
__device__ __forceinline__ uint16_t f2out(float v) {
    return DT == DT_F16 ? f2h_bits(v) : f2bf_bits(v);
}
template <int DT>
__device__ __forceinline__ float in2f(uint32_t b16) {
    return DT == DT_F16 ? h2f((uint16_t)b16) : bf2f(b16);
}

// Byte permute: result byte i = byte sel_i of the 8-byte value {hi:lo}.
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Natural-order activations of one 8-column block, as four 32-bit pairs
// r0=(x0,x1) r1=(x2,x3) r2=(x4,x5) r3=(x6,x7), to kernel order
// (x0,x4) (x1,x5) (x2,x6) (x3,x7).
__device__ __forceinline__ void permute_x8(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3,
                                          uint32_t out[4]) {
    out[0] = perm(r2, r0, 0x05040100u);
    out[1] = perm(r2, r0, 0x07060302u);
    out[2] = perm(r3, r1, 0x05040100u);
    out[3] = perm(r3, r1, 0x07060302u);
}

// Per-group constants used by the unpack routines.
struct ZeroConst {
    uint32_t sub;    // fp16 pair (-(1024+z), -(1024+z)), or unused for bf16
    uint32_t sub16;  // fp16 pair (-(64+z), -(64+z)), or unused for bf16
};

__device__ __forceinline__ ZeroConst make_zero_const_f16(float z) {
    ZeroConst c;
    _Float16 a = (_Float16)(-(1024.0f + z));
    _Float16 b = (_Float16)(-(64.0f + z));
    uint32_t ab = __builtin_bit_cast(uint16_t, a);
    uint32_t bb = __builtin_bit_cast(uint16_t, b);
    c.sub = ab | (ab << 16);
    c.sub16 = bb | (bb << 16);
    return c;
}

// fp16: word -> four pairs of exact codes (u - z) in kernel order.
__device__ __forceinline__ void unpack_f16(uint32_t w, const ZeroConst& zc, uint32_t out[4]) {
    const uint32_t MAGIC = 0x64006400u;                 // 1024.0 in both halves
    const f16x2 inv16 = {(_Float16)0.0625f, (_Float16)0.0625f};
    uint32_t p0 = (w & 0x000F000Fu) | MAGIC;           // 1024 + u0 | 1024 + u4
    uint32_t p1 = (w & 0x00F000F0u) | MAGIC;           // 1024 + 16 u1 | 1024 + 16 u5
    uint32_t w8 = w >> 8;
    uint32_t p2 = (w8 & 0x000F000Fu) | MAGIC;          // 1024 + u2 | 1024 + u6
    uint32_t p3 = (w8 & 0x00F000F0u) | MAGIC;          // 1024 + 16 u3 | 1024 + 16 u7
    f16x2 s = __builtin_bit_cast(f16x2, zc.sub);
    f16x2 s16 = __builtin_bit_cast(f16x2, zc.sub16);
    f16x2 r0 = __builtin_bit_cast(f16x2, p0) + s;
    f16x2 r1 = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, p1), inv16, s16);
    f16x2 r2 = __builtin_bit_cast(f16x2, p2) + s;
    f16x2 r3 = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, p3), inv16, s16);
    out[0] = __builtin_bit_cast(uint32_t, r0);
    out[1] = __builtin_bit_cast(uint32_t, r1);
    out[2] = __builtin_bit_cast(uint32_t, r2);
    out[3] = __builtin_bit_cast(uint32_t, r3);
}

// bf16: word -> four pairs of biased codes 128 + u (exact in bf16), kernel order.
__device__ __forceinline__ void unpack_bf16(uint32_t w, uint32_t out[4]) {
    const uint32_t MAGIC = 0x43004300u;                 // 128.0 in both halves
    out[0] = (w & 0x000F000Fu) | MAGIC;
    out[1] = ((w >> 4) & 0x000F000Fu) | MAGIC;
    out[2] = ((w >> 8) & 0x000F000Fu) | MAGIC;
    out[3] = ((w >> 12) & 0x000F000Fu) | MAGIC;
}

// fp32 += a.x*b.x + a.y*b.y on 16-bit pairs (v_dot2_f32_f16 / v_dot2_f32_bf16).
template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    if constexpr (DT == DT_F16) {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b),
                                      c, false);
    } else {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                               __builtin_bit_cast(bf16x2, b), c, false);
    }
}

// Sum of the two 16-bit values of a pair, in fp32.
template <int DT>
__device__ __forceinline__ float pair_sum(uint32_t p) {
    return in2f<DT>(p & 0xFFFFu) + in2f<DT>(p >> 16);
}

// Group index of input column k: g is a power of two (shift = log2 g) or g == K
// (shift = 31 makes every column group 0).
__device__ __forceinline__ int group_of(int k, int gshift) { return (int)((uint32_t)k >> gshift); }

}  // namespace w4a16
