// 8-bit weight codes (four per 32-bit word, byte k % 4 is element k) as 16-bit MFMA / dot2
// operands in natural pair order, exactly: fp16 takes the byte as a subnormal half u * 2^-24
// (one byte permute per pair); bf16 takes the high half of the code's fp32 conversion
// (exact, the code has at most 8 significant bits).
#pragma once
#include "common.h"

namespace w4a16 {

template <int DT>
__device__ __forceinline__ void codes8(uint32_t w, uint32_t out[2]) {
    if constexpr (DT == DT_F16) {
        out[0] = perm(0u, w, 0x0C010C00u);          // (u0, u1) * 2^-24
        out[1] = perm(0u, w, 0x0C030C02u);          // (u2, u3) * 2^-24
    } else {
        const uint32_t f0 = __float_as_uint((float)(w & 0xFFu));
        const uint32_t f1 = __float_as_uint((float)((w >> 8) & 0xFFu));
        const uint32_t f2 = __float_as_uint((float)((w >> 16) & 0xFFu));
        const uint32_t f3 = __float_as_uint((float)(w >> 24));
        out[0] = perm(f1, f0, 0x07060302u);
        out[1] = perm(f3, f2, 0x07060302u);
    }
}

}  // namespace w4a16
