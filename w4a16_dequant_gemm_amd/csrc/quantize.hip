// Group-wise INT4 quantize-and-pack and the exact fp32 dequantizer.
//
// Quantizer (page "推理优化中“用精度换性能“的核心技术：量化", sections 2.2, 2.3, 3.3 and
// 3.4; page "量化实战深入（GPTQ / AWQ / SmoothQuant / KV 量化）", section 二): per group of g
// consecutive input columns of an output row,
//   asymmetric: s = (max - min)/15, z = round(-min/s), q = clamp(round(x/s) + z, 0, 15);
//   symmetric:  s = max|x|/7, q = clamp(round(x/s), -8, 7), stored as q + 8 with z = 8.
// Every step is IEEE fp32 round-to-nearest-even in a fixed order, the scale is rounded to
// fp16 before it is used (a zero scale becomes 1.0), rounding to integers is
// half-to-even and the zero point is canonicalised to +0.0, so the packed output is
// reproducible bit for bit.
//
// Mapping: one 64-lane wave serves 64/seg groups at once, `seg` lanes per group
// (seg = g/8 when that is a power of two <= 64, else 64 with a loop over the group's
// words).  A lane owns whole 32-bit output words (8 columns), so the pack needs no
// cross-lane traffic; min/max reductions use xor-butterfly shuffles that stay inside
// the aligned lane segment.
#include "common.h"
#include "launch.h"

namespace w4a16 {

template <int SCHEME>
__global__ __launch_bounds__(256) void quantize_pack_kernel(
    const float* __restrict__ W, int N, int K, int g, int G, int seg, int words_per_lane,
    uint32_t* __restrict__ qw, uint16_t* __restrict__ scales, uint16_t* __restrict__ zeros) {
    const int lane = threadIdx.x & 63;
    const long long wave = ((long long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int gpw = 64 / seg;                      // groups served by one wave
    const int slot = lane / seg;
    const int gl = lane % seg;
    const long long gid = (long long)wave * gpw + slot;
    const long long total = (long long)N * G;
    const bool active_group = gid < total;
    const int n = active_group ? (int)(gid / G) : 0;
    const int j = active_group ? (int)(gid % G) : 0;
    const int wcount = g >> 3;                     // words in the group
    const float* row = W + (size_t)n * K + (size_t)j * g;

    float mn = __builtin_inff(), mx = -__builtin_inff();
    for (int it = 0; it < words_per_lane; ++it) {
        const int w = gl + it * seg;
        if (active_group && w < wcount) {
            const float4 a = *reinterpret_cast<const float4*>(row + 8 * w);
            const float4 b = *reinterpret_cast<const float4*>(row + 8 * w + 4);
            if (SCHEME == 0) {
                mn = fminf(mn, fminf(fminf(a.x, a.y), fminf(a.z, a.w)));
                mn = fminf(mn, fminf(fminf(b.x, b.y), fminf(b.z, b.w)));
                mx = fmaxf(mx, fmaxf(fmaxf(a.x, a.y), fmaxf(a.z, a.w)));
                mx = fmaxf(mx, fmaxf(fmaxf(b.x, b.y), fmaxf(b.z, b.w)));
            } else {
                mx = fmaxf(mx, fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))));
                mx = fmaxf(mx, fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
            }
        }
    }
    for (int off = seg >> 1; off > 0; off >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, off, 64));
        mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    }
    if (!active_group) return;

    // Scale (rounded to fp16 and used from then on) and zero point.
    _Float16 sh;
    float s, z;
    rtn_params<SCHEME>(mn, mx, sh, s, z);

    for (int it = 0; it < words_per_lane; ++it) {
        const int w = gl + it * seg;
        if (w < wcount) {
            const float4 a = *reinterpret_cast<const float4*>(row + 8 * w);
            const float4 b = *reinterpret_cast<const float4*>(row + 8 * w + 4);
            const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            uint32_t word = 0;
#pragma unroll
            for (int t = 0; t < 8; ++t) word |= (rtn_code<SCHEME>(x[t], s, z) & 0xFu) << (4 * t);
            qw[(size_t)n * (K >> 3) + (size_t)j * (g >> 3) + w] = word;
        }
    }
    if (gl == 0) {
        scales[(size_t)n * G + j] = __builtin_bit_cast(uint16_t, sh);
        if (zeros) zeros[(size_t)n * G + j] = __builtin_bit_cast(uint16_t, (_Float16)z);
    }
}

__global__ __launch_bounds__(256) void dequantize_kernel(
    const uint32_t* __restrict__ qw, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ zeros, int N, int K, int G, int gshift, float* __restrict__ out) {
    const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const int KW = K >> 3;
    if (idx >= (long long)N * KW) return;
    const int n = (int)(idx / KW);
    const int w = (int)(idx % KW);
    const int j = group_of(8 * w, gshift);
    const float s = h2f(scales[(size_t)n * G + j]);
    const float z = zeros ? h2f(zeros[(size_t)n * G + j]) : 8.0f;
    const uint32_t word = qw[idx];
    float v[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = s * ((float)((word >> (4 * t)) & 0xFu) - z);
    float4* o = reinterpret_cast<float4*>(out + (size_t)n * K + 8 * (size_t)w);
    o[0] = make_float4(v[0], v[1], v[2], v[3]);
    o[1] = make_float4(v[4], v[5], v[6], v[7]);
}

hipError_t launch_quantize_pack(const float* W, int N, int K, int g, int gshift, int scheme,
                                uint32_t* qw, uint16_t* scales, uint16_t* zeros, hipStream_t st) {
    (void)gshift;
    const int G = K / g;
    const int wcount = g / 8;
    const bool pow2 = (wcount & (wcount - 1)) == 0;
    const int seg = (pow2 && wcount <= 64) ? wcount : 64;
    const int words_per_lane = (wcount + seg - 1) / seg;
    const long long groups = (long long)N * G;
    const long long waves = (groups + (64 / seg) - 1) / (64 / seg);
    const long long blocks = (waves + 3) / 4;
    if (scheme == 0)
        hipLaunchKernelGGL(quantize_pack_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, st, W, N,
                           K, g, G, seg, words_per_lane, qw, scales, zeros);
    else
        hipLaunchKernelGGL(quantize_pack_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, st, W, N,
                           K, g, G, seg, words_per_lane, qw, scales, zeros);
    return hipGetLastError();
}

// 8-bit codes (W8A16): the same group-wise RTN with the 8-bit ranges of page
// "推理优化中“用精度换性能“的核心技术：量化", section 3.3 (asymmetric s = (max - min)/255,
// z = rint(-min/s), codes [0, 255]; symmetric s = max|x|/127, codes [-128, 127] stored as
// q + 128), the same fp32 operation order and fp16 scale rounding as the 4-bit kernel.  A
// lane owns whole output words of 4 bytes; byte k % 4 of word k / 4 is element k.
template <int SCHEME>
__device__ __forceinline__ void rtn8_params(float mn, float mx, _Float16& sh, float& s, float& z) {
    const float s32 = (SCHEME == 0) ? (mx - mn) / 255.0f : mx / 127.0f;
    sh = (_Float16)s32;
    s = (float)sh;
    if (s == 0.0f) { s = 1.0f; sh = (_Float16)1.0f; }
    z = (SCHEME == 0) ? (__builtin_rintf((-mn) / s) + 0.0f) : 128.0f;
}

template <int SCHEME>
__device__ __forceinline__ uint32_t rtn8_code(float x, float s, float z) {
    float q;
    if (SCHEME == 0) {
        q = fminf(fmaxf(__builtin_rintf(x / s) + z, 0.0f), 255.0f);
    } else {
        q = fminf(fmaxf(__builtin_rintf(x / s), -128.0f), 127.0f) + 128.0f;
    }
    return (uint32_t)(int)q;
}

template <int SCHEME>
__global__ __launch_bounds__(256) void quantize_pack8_kernel(
    const float* __restrict__ W, int N, int K, int g, int G, int seg, int words_per_lane,
    uint32_t* __restrict__ qw, uint16_t* __restrict__ scales, uint16_t* __restrict__ zeros) {
    const int lane = threadIdx.x & 63;
    const long long wave = ((long long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int gpw = 64 / seg;
    const int slot = lane / seg;
    const int gl = lane % seg;
    const long long gid = (long long)wave * gpw + slot;
    const long long total = (long long)N * G;
    const bool active_group = gid < total;
    const int n = active_group ? (int)(gid / G) : 0;
    const int j = active_group ? (int)(gid % G) : 0;
    const int wcount = g >> 2;                     // 4-code words in the group
    const float* row = W + (size_t)n * K + (size_t)j * g;
    float mn = __builtin_inff(), mx = -__builtin_inff();
    for (int it = 0; it < words_per_lane; ++it) {
        const int w = gl + it * seg;
        if (active_group && w < wcount) {
            const float4 a = *reinterpret_cast<const float4*>(row + 4 * w);
            if (SCHEME == 0) {
                mn = fminf(mn, fminf(fminf(a.x, a.y), fminf(a.z, a.w)));
                mx = fmaxf(mx, fmaxf(fmaxf(a.x, a.y), fmaxf(a.z, a.w)));
            } else {
                mx = fmaxf(mx, fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))));
            }
        }
    }
    for (int off = seg >> 1; off > 0; off >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, off, 64));
        mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    }
    if (!active_group) return;
    _Float16 sh;
    float s, z;
    rtn8_params<SCHEME>(mn, mx, sh, s, z);
    for (int it = 0; it < words_per_lane; ++it) {
        const int w = gl + it * seg;
        if (w < wcount) {
            const float4 a = *reinterpret_cast<const float4*>(row + 4 * w);
            const uint32_t word = rtn8_code<SCHEME>(a.x, s, z) | (rtn8_code<SCHEME>(a.y, s, z) << 8) |
                                  (rtn8_code<SCHEME>(a.z, s, z) << 16) | (rtn8_code<SCHEME>(a.w, s, z) << 24);
            qw[(size_t)n * (K >> 2) + (size_t)j * (g >> 2) + w] = word;
        }
    }
    if (gl == 0) {
        scales[(size_t)n * G + j] = __builtin_bit_cast(uint16_t, sh);
        if (zeros) zeros[(size_t)n * G + j] = __builtin_bit_cast(uint16_t, (_Float16)z);
    }
}

hipError_t launch_quantize_pack8(const float* W, int N, int K, int g, int scheme, uint32_t* qw,
                                 uint16_t* scales, uint16_t* zeros, hipStream_t st) {
    const int G = K / g;
    const int wcount = g / 4;
    const bool pow2 = (wcount & (wcount - 1)) == 0;
    const int seg = (pow2 && wcount <= 64) ? wcount : 64;
    const int words_per_lane = (wcount + seg - 1) / seg;
    const long long groups = (long long)N * G;
    const long long waves = (groups + (64 / seg) - 1) / (64 / seg);
    const long long blocks = (waves + 3) / 4;
    if (scheme == 0)
        hipLaunchKernelGGL(quantize_pack8_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, st, W, N, K, g, G,
                           seg, words_per_lane, qw, scales, zeros);
    else
        hipLaunchKernelGGL(quantize_pack8_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, st, W, N, K, g, G,
                           seg, words_per_lane, qw, scales, zeros);
    return hipGetLastError();
}

hipError_t launch_dequantize(const uint32_t* qw, const uint16_t* scales, const uint16_t* zeros,
                             int N, int K, int g, int gshift, float* out, hipStream_t st) {
    const long long words = (long long)N * (K / 8);
    const long long blocks = (words + 255) / 256;
    hipLaunchKernelGGL(dequantize_kernel, dim3((unsigned)blocks), dim3(256), 0, st, qw, scales,
                       zeros, N, K, K / g, gshift, out);
    return hipGetLastError();
}

}  // namespace w4a16
