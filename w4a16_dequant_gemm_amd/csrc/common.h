// Device-side building blocks shared by the W4A16 kernels (gfx950 / CDNA4, wave64).
//
// Code layout.  A 32-bit word of the packed weight row holds 8 consecutive input
// columns k0..k7, element k_t in bits 4t..4t+3.  The kernels never rebuild the natural
// column order: a word is split into four 32-bit registers, each holding two codes in
// its two 16-bit halves, with one or two integer instructions per register.  The
// activations are permuted the same way once, when they are loaded, so every
// dot product / MFMA sees matching pairs (a dot product is invariant under a
// permutation of k applied to both operands).
//
// Dequantization x_hat = s * (u - z) (page "推理优化中“用精度换性能“的核心技术：量化",
// section 2.3; page "量化实战深入（GPTQ / AWQ / SmoothQuant / KV 量化）", section 二) is
// split so that no rounded 16-bit weight is ever formed:
//   sum_k x_k s (u_k - z) = s * ( sum_k x_k u_k  -  z * sum_k x_k ),
// the first sum is computed by v_dot2 / MFMA on exact codes, the activation sum is
// computed once per chunk or group, and the per-group scale multiplies the fp32 result.
// Exact codes in a 16-bit float:
//   fp16: a nibble u in the low bits of an fp16 with zero exponent is the subnormal
//     u * 2^-24; both v_dot2_f32_f16 and the fp16 MFMAs multiply subnormals exactly, so
//     masking alone yields the operand (products are exact in fp32).  A nibble at bits
//     4..7 is still subnormal (16u * 2^-24), which the GEMV uses to skip a shift.
//   bf16: bf16 subnormals would push the fp32 products below the normal range, so the
//     nibble is OR-ed into the mantissa of 128.0 (0x4300), giving 128 + u exactly; the
//     bias 128 is removed with the activation sum: s * (sum x (128+u) - (128+z) sum x).
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
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

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

// RTN group parameters (fp32, round-to-nearest-even, this order): asymmetric from the
// group's min and max, s = fp16((max - min) / 15) (1.0 if that is 0), z = rint(-min/s) + 0;
// symmetric from max|x|, s = fp16(max|x| / 7), z = 8 (offset-binary storage).
template <int SCHEME>
__device__ __forceinline__ void rtn_params(float mn, float mx, _Float16& sh, float& s, float& z) {
    const float s32 = (SCHEME == 0) ? (mx - mn) / 15.0f : mx / 7.0f;
    sh = (_Float16)s32;
    s = (float)sh;
    if (s == 0.0f) { s = 1.0f; sh = (_Float16)1.0f; }
    z = (SCHEME == 0) ? (__builtin_rintf((-mn) / s) + 0.0f) : 8.0f;
}

// The stored 4-bit code of x with those parameters: clamp(rint(x/s) + z, 0, 15), or
// clamp(rint(x/s), -8, 7) + 8 for the symmetric scheme.
template <int SCHEME>
__device__ __forceinline__ uint32_t rtn_code(float x, float s, float z) {
    float q;
    if (SCHEME == 0) {
        q = __builtin_rintf(x / s) + z;
        q = fminf(fmaxf(q, 0.0f), 15.0f);
    } else {
        q = __builtin_rintf(x / s);
        q = fminf(fmaxf(q, -8.0f), 7.0f) + 8.0f;
    }
    return (uint32_t)(int)q;
}

// Byte permute: result byte i = byte sel_i of the 8-byte value {hi:lo}.
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Natural-order activations of one 8-column block, as four 32-bit pairs
// r0=(x0,x1) r1=(x2,x3) r2=(x4,x5) r3=(x6,x7), to "mask order"
// (x0,x4) (x1,x5) (x2,x6) (x3,x7) -- the pair order of unpack_mask_f16.
__device__ __forceinline__ void permute_x8(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3,
                                          uint32_t out[4]) {
    out[0] = perm(r2, r0, 0x05040100u);
    out[1] = perm(r2, r0, 0x07060302u);
    out[2] = perm(r3, r1, 0x05040100u);
    out[3] = perm(r3, r1, 0x07060302u);
}

// Natural order to "byte order" (x0,x2) (x4,x6) (x1,x3) (x5,x7) -- the pair order of
// unpack_byte.
__device__ __forceinline__ void permute_x8_byte(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3,
                                               uint32_t out[4]) {
    out[0] = perm(r1, r0, 0x05040100u);   // x0, x2
    out[1] = perm(r3, r2, 0x05040100u);   // x4, x6
    out[2] = perm(r1, r0, 0x07060302u);   // x1, x3
    out[3] = perm(r3, r2, 0x07060302u);   // x5, x7
}

// fp16, GEMV form: four registers of subnormal codes in mask order,
// (u0,u4) (16u1,16u5) (u2,u6) (16u3,16u7) times 2^-24.  Five integer instructions.
__device__ __forceinline__ void unpack_mask_f16(uint32_t w, uint32_t out[4]) {
    const uint32_t w8 = w >> 8;
    out[0] = w & 0x000F000Fu;
    out[1] = w & 0x00F000F0u;
    out[2] = w8 & 0x000F000Fu;
    out[3] = w8 & 0x00F000F0u;
}

// Byte form for either dtype: codes in byte order (u0,u2) (u4,u6) (u1,u3) (u5,u7), each
// half = MAGIC_HI byte : code byte.  MAGIC = 0 gives fp16 subnormals u * 2^-24,
// MAGIC = 0x43 gives bf16 128 + u.  Seven instructions (two masks, one shift, four
// byte permutes).
template <uint32_t MAGIC>
__device__ __forceinline__ void unpack_byte(uint32_t w, uint32_t out[4]) {
    const uint32_t t0 = w & 0x0F0F0F0Fu;           // u0 u2 u4 u6
    const uint32_t t1 = (w >> 4) & 0x0F0F0F0Fu;    // u1 u3 u5 u7
    const uint32_t mag = MAGIC * 0x01010101u;
    // selector bytes 0..3 pick from the low operand, 4..7 from the high operand
    out[0] = perm(mag, t0, 0x04010400u);
    out[1] = perm(mag, t0, 0x04030402u);
    out[2] = perm(mag, t1, 0x04010400u);
    out[3] = perm(mag, t1, 0x04030402u);
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL,
                                                             0xF, 0xF, true));
}

// Sum over a 64-lane wave with DPP row operations; the total is returned in every lane.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_mov<0x141>(v);   // row_half_mirror
    v += dpp_mov<0x140>(v);   // row_mirror: every lane holds its 16-lane row sum
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (r0 + r1) + (r2 + r3);
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

// Scales and zeros of `rows` consecutive weight rows into LDS, groups [g0, g0 + gl) of each, as
// (s | z << 16) dwords at a row stride of gp dwords (odd: the 16 or 32 rows a wave reads at one
// group fall in distinct banks).  REP threads per row: thread t < REP rows stages pieces
// t / rows, t / rows + REP, ... of row min(row0 + t % rows, N - 1), a piece being the 16 bytes
// at local offset min(8 p, gl - 8) (inside the row's range, the last one overlapping its
// neighbour), all of a thread's loads in flight at once (gl <= 8 PIECES); 2-byte loads
// by one thread per row when gl < 8.  Without zeros (hz false) the high halves are 0.  The
// caller synchronizes before reading.  Staged once per block, this replaces two 2-byte loads
// per row set and k-step, each touching as many cache lines as the row set has rows.
constexpr int kSzStagePieces = 12;
template <int REP, int PIECES = kSzStagePieces>
__device__ __forceinline__ void stage_sz_rows(uint32_t* szl, int gp, int tid, int rows, int row0, int N,
                                              int G, int g0, int gl, bool hz, __amdgpu_buffer_rsrc_t rs,
                                              __amdgpu_buffer_rsrc_t rz, __amdgpu_buffer_rsrc_t rnull) {
    constexpr int PT = (PIECES + REP - 1) / REP;                  // pieces per thread
    if (tid >= REP * rows) return;
    const int rr = tid % rows, k = tid / rows;
    const int row = min(row0 + rr, N - 1);
    const int rbase = (row * G + g0) * 2;
    uint32_t* dst = szl + rr * gp;
    if (gl >= 8) {
        const int P = (gl + 7) >> 3;
        u32x4 sv[PT], zv[PT];
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int p = k + REP * i;
            const int o = rbase + 2 * min(8 * p, gl - 8);
            sv[i] = __builtin_amdgcn_raw_buffer_load_b128(p < P ? rs : rnull, o, 0, 0);
            zv[i] = __builtin_amdgcn_raw_buffer_load_b128(p < P && hz ? rz : rnull, o, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int p = k + REP * i;
            if (p < P) {
                uint32_t* d = dst + min(8 * p, gl - 8);
                const uint32_t sw[4] = {sv[i].x, sv[i].y, sv[i].z, sv[i].w};
                const uint32_t zw[4] = {zv[i].x, zv[i].y, zv[i].z, zv[i].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    d[2 * j] = (sw[j] & 0xFFFFu) | (zw[j] << 16);
                    d[2 * j + 1] = (sw[j] >> 16) | (zw[j] & 0xFFFF0000u);
                }
            }
        }
    } else if (k == 0) {
        for (int j = 0; j < gl; ++j) {
            const uint32_t sj = __builtin_amdgcn_raw_buffer_load_b16(rs, rbase + 2 * j, 0, 0);
            const uint32_t zj = hz ? __builtin_amdgcn_raw_buffer_load_b16(rz, rbase + 2 * j, 0, 0) : 0u;
            dst[j] = sj | (zj << 16);
        }
    }
}

}  // namespace w4a16
