// KV-cache quantization (KV8 / KV4, one scale per (head, token) row) and the decode attention
// that streams the quantized cache.
//
// Method (page "量化实战深入（GPTQ / AWQ / SmoothQuant / KV 量化）", 六 KV Cache 量化: keys and
// values quantized separately, per token, KV8 / KV4, to fit more concurrent requests; page
// "Quantization & Acceleration: 解释 W8A8 与 W4A16 的差异与取舍", 深度剖析 ③: W4A16 + KV INT8).
// KV8: s = fp16(max|x| / 127) (1 if 0), codes clamp(rint(x / s), -127, 127) (fp32, stored
// scale); KV4: the asymmetric RTN of the weight quantizer with g = D.  Cache layout
// [Hkv, Tmax, D] (a head's tokens contiguous), scales / zeros [Hkv, Tmax] fp16.
//
// Decode attention, out[h] = softmax(q_h K^T / sqrt(D)) V over the first T tokens of kv head
// h / (Hq / Hkv), in two launches (split over tokens, then a merge):
//   split kernel, block (split, h), 256 threads: each thread scores whole tokens (its key row
//   read with 16-byte loads, codes converted in registers, q in registers), the block takes
//   its max and the exponentials, then every wave accumulates p_t * value row for a quarter
//   of the tokens with one lane per pair of dimensions (a value row is one coalesced read);
//   the partial (max, sum, unnormalized output) goes to the workspace;
//   merge kernel: rescales the splits to the common max and normalizes.
// Dequantization happens in registers only; the cache is read once.
#include "common.h"
#include "launch.h"

namespace w4a16 {

namespace {

constexpr int kKvThreads = 256;
constexpr int kKvChunkMax = 2048;       // tokens per split (LDS scores)

// Quantize rows of D values: lane owns 8 consecutive values; D / 8 lanes per row.
template <int DT, int BITS, int D>
__global__ __launch_bounds__(256) void kv_quant_kernel(const uint16_t* __restrict__ x, long long rows,
                                                       void* __restrict__ codes, uint16_t* __restrict__ scales,
                                                       uint16_t* __restrict__ zeros) {
    constexpr int SEG = D / 8;
    const int lane = threadIdx.x & 63;
    const long long row = ((long long)blockIdx.x * 256 + threadIdx.x) / SEG;
    const int gl = lane % SEG;
    const bool live = row < rows;
    const long long r = live ? row : 0;
    const u32x4 raw = *reinterpret_cast<const u32x4*>(x + r * D + 8 * gl);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = in2f<DT>((w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
    float mn = __builtin_inff(), mx = BITS == 8 ? 0.0f : -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (BITS == 8) mx = fmaxf(mx, fabsf(v[i]));
        else { mn = fminf(mn, v[i]); mx = fmaxf(mx, v[i]); }
    }
    for (int off = SEG >> 1; off > 0; off >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, off, 64));
        mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    }
    if (!live) return;
    if constexpr (BITS == 8) {
        const _Float16 sh = (_Float16)(mx / 127.0f);
        float s = (float)sh;
        _Float16 sh_out = sh;
        if (s == 0.0f) { s = 1.0f; sh_out = (_Float16)1.0f; }
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float c = fminf(fmaxf(__builtin_rintf(v[i] / s), -127.0f), 127.0f);
            const uint32_t b = (uint32_t)(int)c & 0xFFu;
            if (i < 4) lo |= b << (8 * i); else hi |= b << (8 * (i - 4));
        }
        *reinterpret_cast<uint2*>(static_cast<int8_t*>(codes) + r * D + 8 * gl) = make_uint2(lo, hi);
        if (gl == 0) scales[r] = __builtin_bit_cast(uint16_t, sh_out);
    } else {
        _Float16 sh;
        float s, z;
        rtn_params<0>(mn, mx, sh, s, z);
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) word |= (rtn_code<0>(v[i], s, z) & 0xFu) << (4 * i);
        static_cast<uint32_t*>(codes)[r * (D / 8) + gl] = word;
        if (gl == 0) {
            scales[r] = __builtin_bit_cast(uint16_t, sh);
            zeros[r] = __builtin_bit_cast(uint16_t, (_Float16)z);
        }
    }
}

// the 8 codes of a 32-bit word (KV4, as floats) or of 8 bytes (KV8)
template <int BITS>
__device__ __forceinline__ void codes8(uint32_t a, uint32_t b, float c[8]) {
    if constexpr (BITS == 8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            c[i] = (float)(int)(signed char)(a >> (8 * i));
            c[4 + i] = (float)(int)(signed char)(b >> (8 * i));
        }
    } else {
        (void)b;
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = (float)((a >> (4 * i)) & 0xFu);
    }
}

template <int DT, int BITS, int D>
__global__ __launch_bounds__(kKvThreads) void kv_attn_split_kernel(
    const uint16_t* __restrict__ q, int Hq, int Hkv, int T, int Tmax, int chunk,
    const void* __restrict__ kc, const uint16_t* __restrict__ ks, const uint16_t* __restrict__ kz,
    const void* __restrict__ vc, const uint16_t* __restrict__ vs, const uint16_t* __restrict__ vz,
    float* __restrict__ part) {
    constexpr int RB = BITS == 8 ? D : D / 2;          // bytes per cached row
    __shared__ float sc[kKvChunkMax];
    __shared__ float red[kKvThreads];
    __shared__ float acc_w[4][D];
    const int split = blockIdx.x;
    const int h = blockIdx.y;
    const int nsplit = gridDim.x;
    const int kvh = h / (Hq / Hkv);
    const int tid = threadIdx.x;
    const int t0 = split * chunk;
    const int t1 = min(T, t0 + chunk);
    const int n = max(0, t1 - t0);
    const long long rowbase = (long long)kvh * Tmax;
    // q in registers (fp32) and its sum (for the KV4 zero point)
    float qv[D];
#pragma unroll
    for (int d = 0; d < D; ++d) qv[d] = in2f<DT>(q[(long long)h * D + d]);
    float qsum = 0.0f;
    if constexpr (BITS == 4) {
#pragma unroll
        for (int d = 0; d < D; ++d) qsum += qv[d];
    }
    const float rsd = 1.0f / sqrtf((float)D);
    // 1. scores of this split, one thread per token
    float mloc = -__builtin_inff();
    for (int i = tid; i < n; i += kKvThreads) {
        const long long row = rowbase + t0 + i;
        const unsigned char* kr = static_cast<const unsigned char*>(kc) + row * RB;
        float dot = 0.0f;
#pragma unroll
        for (int p = 0; p < RB / 16; ++p) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(kr + 16 * p);
            float c[8];
            if constexpr (BITS == 8) {
                codes8<8>(w.x, w.y, c);
#pragma unroll
                for (int e = 0; e < 8; ++e) dot = fmaf(qv[16 * p + e], c[e], dot);
                codes8<8>(w.z, w.w, c);
#pragma unroll
                for (int e = 0; e < 8; ++e) dot = fmaf(qv[16 * p + 8 + e], c[e], dot);
            } else {
                const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    codes8<4>(ww[k], 0u, c);
#pragma unroll
                    for (int e = 0; e < 8; ++e) dot = fmaf(qv[32 * p + 8 * k + e], c[e], dot);
                }
            }
        }
        const float s = h2f(ks[row]);
        float score;
        if constexpr (BITS == 8) score = dot * s * rsd;
        else score = (dot - h2f(kz[row]) * qsum) * s * rsd;
        sc[i] = score;
        mloc = fmaxf(mloc, score);
    }
    red[tid] = mloc;
    __syncthreads();
    for (int w = kKvThreads / 2; w > 0; w >>= 1) {
        if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
        __syncthreads();
    }
    const float m = red[0];
    __syncthreads();
    float lsum = 0.0f;
    for (int i = tid; i < n; i += kKvThreads) {
        const float p = expf(sc[i] - m);
        sc[i] = p;
        lsum += p;
    }
    red[tid] = lsum;
    __syncthreads();
    for (int w = kKvThreads / 2; w > 0; w >>= 1) {
        if (tid < w) red[tid] += red[tid + w];
        __syncthreads();
    }
    const float l = red[0];
    // 2. p V: wave w takes tokens w, w + 4, ...; lane owns dimensions 2 lane, 2 lane + 1 (D = 128)
    //    or lane (D = 64)
    const int wave = tid >> 6;
    const int lane = tid & 63;
    constexpr int DPL = D / 64;                      // dimensions per lane
    float acc[DPL];
#pragma unroll
    for (int j = 0; j < DPL; ++j) acc[j] = 0.0f;
    for (int i = wave; i < n; i += 4) {
        const long long row = rowbase + t0 + i;
        const float ps = sc[i] * h2f(vs[row]);
        const unsigned char* vr = static_cast<const unsigned char*>(vc) + row * RB;
        if constexpr (BITS == 8) {
            if constexpr (DPL == 2) {
                const uint32_t two = *reinterpret_cast<const uint16_t*>(vr + 2 * lane);
                acc[0] = fmaf(ps, (float)(int)(signed char)two, acc[0]);
                acc[1] = fmaf(ps, (float)(int)(signed char)(two >> 8), acc[1]);
            } else {
                acc[0] = fmaf(ps, (float)(int)(signed char)vr[lane], acc[0]);
            }
        } else {
            const float z = h2f(vz[row]);
            if constexpr (DPL == 2) {
                const uint32_t b = vr[lane];
                acc[0] = fmaf(ps, (float)(b & 0xFu) - z, acc[0]);
                acc[1] = fmaf(ps, (float)(b >> 4) - z, acc[1]);
            } else {
                const uint32_t b = vr[lane >> 1];
                acc[0] = fmaf(ps, (float)((b >> (4 * (lane & 1))) & 0xFu) - z, acc[0]);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < DPL; ++j) acc_w[wave][DPL * lane + j] = acc[j];
    __syncthreads();
    float* out = part + ((long long)h * nsplit + split) * (D + 2);
    for (int d = tid; d < D; d += kKvThreads) out[2 + d] = acc_w[0][d] + acc_w[1][d] + acc_w[2][d] + acc_w[3][d];
    if (tid == 0) {
        out[0] = n > 0 ? m : -__builtin_inff();
        out[1] = l;
    }
}

template <int DT, int D>
__global__ __launch_bounds__(256) void kv_attn_merge_kernel(const float* __restrict__ part, int nsplit,
                                                            uint16_t* __restrict__ out) {
    const int h = blockIdx.x;
    const float* p = part + (long long)h * nsplit * (D + 2);
    float m = -__builtin_inff();
    for (int j = 0; j < nsplit; ++j) m = fmaxf(m, p[j * (D + 2)]);
    float l = 0.0f;
    for (int j = 0; j < nsplit; ++j) {
        const float mj = p[j * (D + 2)];
        if (mj != -__builtin_inff()) l += p[j * (D + 2) + 1] * expf(mj - m);
    }
    for (int d = threadIdx.x; d < D; d += 256) {
        float o = 0.0f;
        for (int j = 0; j < nsplit; ++j) {
            const float mj = p[j * (D + 2)];
            if (mj != -__builtin_inff()) o += p[j * (D + 2) + 2 + d] * expf(mj - m);
        }
        out[(long long)h * D + d] = f2out<DT>(o / l);
    }
}

int kv_splits(int Hq, int T) {
    int ns = (1024 + Hq - 1) / Hq;                     // about four blocks per CU in all
    ns = min(ns, (T + 63) / 64);                        // at least 64 tokens per split
    ns = max(ns, (T + kKvChunkMax - 1) / kKvChunkMax);  // at most kKvChunkMax per split
    return max(ns, 1);
}

template <int DT, int BITS, int D>
hipError_t kv_attn(const void* q, int Hq, int Hkv, int T, int Tmax, const void* kc, const uint16_t* ks,
                   const uint16_t* kz, const void* vc, const uint16_t* vs, const uint16_t* vz, float* work,
                   void* out, hipStream_t st) {
    const int ns = kv_splits(Hq, T);
    const int chunk = (T + ns - 1) / ns;
    hipLaunchKernelGGL((kv_attn_split_kernel<DT, BITS, D>), dim3(ns, Hq), dim3(kKvThreads), 0, st,
                       static_cast<const uint16_t*>(q), Hq, Hkv, T, Tmax, chunk, kc, ks, kz, vc, vs, vz, work);
    hipLaunchKernelGGL((kv_attn_merge_kernel<DT, D>), dim3(Hq), dim3(256), 0, st, work, ns,
                       static_cast<uint16_t*>(out));
    return hipGetLastError();
}

template <int DT, int BITS>
hipError_t kv_quant(const void* x, long long rows, int D, void* codes, uint16_t* scales, uint16_t* zeros,
                    hipStream_t st) {
    const unsigned blocks = (unsigned)((rows * (D / 8) + 255) / 256);
    if (D == 64)
        hipLaunchKernelGGL((kv_quant_kernel<DT, BITS, 64>), dim3(blocks), dim3(256), 0, st,
                           static_cast<const uint16_t*>(x), rows, codes, scales, zeros);
    else
        hipLaunchKernelGGL((kv_quant_kernel<DT, BITS, 128>), dim3(blocks), dim3(256), 0, st,
                           static_cast<const uint16_t*>(x), rows, codes, scales, zeros);
    return hipGetLastError();
}

}  // namespace

long long kv_attention_workspace_floats(long long Hq, long long T, long long D) {
    return Hq * kv_splits((int)Hq, (int)T) * (D + 2);
}

hipError_t launch_kv_quantize(const void* x, int dtype, long long rows, int D, int bits, void* codes,
                              uint16_t* scales, uint16_t* zeros, hipStream_t st) {
    if (dtype == DT_F16)
        return bits == 8 ? kv_quant<DT_F16, 8>(x, rows, D, codes, scales, zeros, st)
                         : kv_quant<DT_F16, 4>(x, rows, D, codes, scales, zeros, st);
    return bits == 8 ? kv_quant<DT_BF16, 8>(x, rows, D, codes, scales, zeros, st)
                     : kv_quant<DT_BF16, 4>(x, rows, D, codes, scales, zeros, st);
}

hipError_t launch_kv_attention(const void* q, int dtype, int Hq, int Hkv, int T, int Tmax, int D, int bits,
                               const void* kc, const uint16_t* ks, const uint16_t* kz, const void* vc,
                               const uint16_t* vs, const uint16_t* vz, float* work, void* out, hipStream_t st) {
#define W4A16_KV_CASE(DTV, BV, DV)                                                                          \
    if (dtype == DTV && bits == BV && D == DV)                                                              \
        return kv_attn<DTV, BV, DV>(q, Hq, Hkv, T, Tmax, kc, ks, kz, vc, vs, vz, work, out, st);
    W4A16_KV_CASE(DT_F16, 8, 64)
    W4A16_KV_CASE(DT_F16, 8, 128)
    W4A16_KV_CASE(DT_F16, 4, 64)
    W4A16_KV_CASE(DT_F16, 4, 128)
    W4A16_KV_CASE(DT_BF16, 8, 64)
    W4A16_KV_CASE(DT_BF16, 8, 128)
    W4A16_KV_CASE(DT_BF16, 4, 64)
    W4A16_KV_CASE(DT_BF16, 4, 128)
#undef W4A16_KV_CASE
    return hipErrorInvalidValue;
}

}  // namespace w4a16
