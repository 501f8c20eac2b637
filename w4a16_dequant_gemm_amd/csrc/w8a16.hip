// W8A16 decode kernel: the weight-only linear layer with 8-bit codes (four per 32-bit word,
// byte k % 4 of word k / 4 is element k) and the same fp16 scale and zero point per group
// of g input columns (page "大模型推理中 Weight-only、W8A8 和 FP8 量化有什么区别？如何选型？",
// section 二, INT8 / INT4 weight-only with 16-bit activations; page "推理优化中“用精度换性能“
// 的核心技术：量化", section 3.3 for the 8-bit ranges).
//
// Y[m, n] = sum_g s[n, g] (sum_{k in g} x[m, k] u[n, k] - z[n, g] sum_{k in g} x[m, k]).
//
// Mapping: blocks of 8 waves; each wave owns one output row (two from M = 2 on, so that each
// activation read from LDS serves both) and its lanes stream the row in 16-byte loads (a 1 KB
// contiguous run per wave instruction), lane l taking the 16-column chunks l, l + 64, ... of
// each slice; eight loads in flight per lane.  The block stages its
// activations in LDS in natural order with the 16-column chunk sums, the whole row of K at
// once while M rows fit 64 KB, else in K slices of a multiple of 1024 columns.  Codes: fp16 activations take the code bytes as subnormal halves u * 2^-24 (one
// byte permute per pair, exact) and v_dot2; bf16 activations take each code as an exact bf16
// (the high half of its fp32 conversion) and v_dot2.  Per chunk the group factors fold the
// dot product and the chunk's activation sum: fp16 s' = s * 2^24, c = -z * s' (products and
// sums in units of 2^-24); bf16 s' = s, c = -z * s.  One DPP reduction per row.
#include "common.h"
#include "launch.h"
#include "w8.h"

namespace w4a16 {

namespace {

constexpr int kW8Waves = 8;
constexpr int kW8Threads = 64 * kW8Waves;
constexpr int kW8Unroll = 8;                // 16-byte weight loads in flight per lane
constexpr int kW8LdsBudget = 65536;         // staged activations and chunk sums
constexpr int kW8MaxM = 16;
#ifndef W4A16_W8_TWO_ROW_MIN_M
#define W4A16_W8_TWO_ROW_MIN_M 2
#endif
// from this many activation rows on each wave owns two weight rows, so that every activation
// read from LDS serves both (LDS reads per weight byte grow with M and at M = 4 match the
// CU's share of the HBM stream)
constexpr int kW8TwoRowMinM = W4A16_W8_TWO_ROW_MIN_M;

__host__ __device__ constexpr long long w8_lds_bytes(int M, int K) {
    return (long long)M * K * 2 + (long long)M * (K / 16) * 4;
}

template <int DT, int M, int R>
__global__ __launch_bounds__(kW8Threads) void gemv8_kernel(
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ qw, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ zeros, int has_zeros, uint16_t* __restrict__ Y, int N, int K, int G,
    int gshift, int KS) {
    extern __shared__ __attribute__((aligned(16))) uint32_t lds8[];
    constexpr int U = kW8Unroll / R;                       // chunks per row and batch
    const int CS = KS >> 4;                                // 16-column chunks per slice
    const int KPS = KS >> 3;                               // 8-column pieces per slice row (even)
    u32x4* xs = reinterpret_cast<u32x4*>(lds8);             // [M][2][KS / 16] pieces of 8 columns
    float* csum = reinterpret_cast<float*>(lds8 + (size_t)M * (KS >> 1));   // [M][CS]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // R consecutive output rows per wave; rows past the last one re-read row N - 1 (valid
    // memory, never stored), and every wave stages and meets the barriers
    const int row0 = (blockIdx.x * kW8Waves + wave) * R;
    int rrow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) rrow[r] = min(row0 + r, N - 1);
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(qw), 0, N * K, 0x00020000);
    const uint16_t* zsrc = has_zeros ? zeros : scales;
    const uint32_t one2 = DT == DT_F16 ? 0x3C003C00u : 0x3F803F80u;
    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

    for (int k0 = 0; k0 < K; k0 += KS) {
        const int ks = min(KS, K - k0);                    // columns in this slice (multiple of 32)
        const int kp = ks >> 3;
        // 1. Stage the slice's activations (natural order) and 16-column chunk sums; every
        //    thread runs every round, so the pair exchange and the barriers are uniform.
        if (k0 > 0) __syncthreads();                       // the previous slice is consumed
        const int pieces = M * kp;
        for (int p0 = 0; p0 < pieces; p0 += kW8Threads) {
            const int p = p0 + tid;
            const bool ok = p < pieces;
            const int m = ok ? p / kp : 0;
            const int c8 = ok ? p % kp : 0;
            const u32x4 v = ok ? *reinterpret_cast<const u32x4*>(X + (size_t)m * K + k0 + 8 * (size_t)c8)
                               : u32x4{0u, 0u, 0u, 0u};
            // even pieces in the first half of the row's slots, odd ones in the second, so the
            // lanes of a wave read consecutive 16-byte slots (no bank conflicts)
            if (ok) xs[m * KPS + (c8 & 1) * (KPS >> 1) + (c8 >> 1)] = v;
            float sum = dot2<DT>(v.x, one2, 0.0f);
            sum = dot2<DT>(v.y, one2, sum);
            sum = dot2<DT>(v.z, one2, sum);
            sum = dot2<DT>(v.w, one2, sum);
            sum += __shfl_xor(sum, 1, 64);                // pieces 2c and 2c + 1 form chunk c
            if (ok && (c8 & 1) == 0) csum[m * CS + (c8 >> 1)] = DT == DT_F16 ? sum * 5.9604644775390625e-8f : sum;
        }
        __syncthreads();

        // 2. The rows' chunks of this slice.  Chunks past the slice re-read its last chunk
        //    (valid memory, result unused).  Each activation read from LDS serves all R rows.
        const int cs = ks >> 4;
        const int cpl = (cs + 63) >> 6;
        for (int cb = 0; cb < cpl; cb += U) {
            u32x4 w[U][R];
            uint16_t sb[U][R], zb[U][R];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = min(lane + 64 * (cb + u), cs - 1);
                const int grp = (k0 + 16 * c) >> gshift;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    w[u][r] = __builtin_amdgcn_raw_buffer_load_b128(rw, rrow[r] * K + k0 + 16 * c, 0, 2 /* nt */);
                    sb[u][r] = scales[(size_t)rrow[r] * G + grp];
                    zb[u][r] = zsrc[(size_t)rrow[r] * G + grp];
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = lane + 64 * (cb + u);
                if (c < cs) {
                    float sp[R], cz[R];
                    uint32_t cd[R][8];
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const float sv = h2f(sb[u][r]);
                        const float zv = has_zeros ? h2f(zb[u][r]) : 128.0f;
                        sp[r] = DT == DT_F16 ? sv * 16777216.0f : sv;
                        cz[r] = -zv * sp[r];
                        codes8<DT>(w[u][r].x, &cd[r][0]);
                        codes8<DT>(w[u][r].y, &cd[r][2]);
                        codes8<DT>(w[u][r].z, &cd[r][4]);
                        codes8<DT>(w[u][r].w, &cd[r][6]);
                    }
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        const u32x4 a0 = xs[m * KPS + c];
                        const u32x4 a1 = xs[m * KPS + (KPS >> 1) + c];
                        const float cm = csum[m * CS + c];
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            float pd = dot2<DT>(a0.x, cd[r][0], 0.0f);
                            pd = dot2<DT>(a0.y, cd[r][1], pd);
                            pd = dot2<DT>(a0.z, cd[r][2], pd);
                            pd = dot2<DT>(a0.w, cd[r][3], pd);
                            pd = dot2<DT>(a1.x, cd[r][4], pd);
                            pd = dot2<DT>(a1.y, cd[r][5], pd);
                            pd = dot2<DT>(a1.z, cd[r][6], pd);
                            pd = dot2<DT>(a1.w, cd[r][7], pd);
                            acc[r][m] = fmaf(cz[r], cm, fmaf(sp[r], pd, acc[r][m]));
                        }
                    }
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const float v = wave_sum(acc[r][m]);
            if (row0 + r < N && lane == 0) Y[(size_t)m * N + row0 + r] = f2out<DT>(v);
        }
}

// Slice width: the whole row while M rows of activations and their chunk sums fit the LDS
// budget, else the largest multiple of 1024 columns that does.
int w8_slice(int M, int K) {
    if (w8_lds_bytes(M, K) <= kW8LdsBudget) return K;
    int ks = (int)((4LL * kW8LdsBudget) / (9LL * M)) / 1024 * 1024;    // 2.25 bytes per column and row
    while (ks > 1024 && w8_lds_bytes(M, ks) > kW8LdsBudget) ks -= 1024;
    return ks;
}

template <int DT, int M>
hipError_t run_gemv8(const LinearArgs& a, hipStream_t st) {
    const int ks = w8_slice(M, a.K);
    const long long lds = w8_lds_bytes(M, ks);
    if (M >= kW8TwoRowMinM) {
        const long long blocks = (a.N + 2 * kW8Waves - 1) / (2 * kW8Waves);
        hipLaunchKernelGGL((gemv8_kernel<DT, M, 2>), dim3((unsigned)blocks), dim3(kW8Threads), (size_t)lds, st,
                           static_cast<const uint16_t*>(a.X), a.qw, a.scales, a.zeros, a.zeros ? 1 : 0,
                           static_cast<uint16_t*>(a.Y), a.N, a.K, a.G, a.gshift, ks);
    } else {
        const long long blocks = (a.N + kW8Waves - 1) / kW8Waves;
        hipLaunchKernelGGL((gemv8_kernel<DT, M, 1>), dim3((unsigned)blocks), dim3(kW8Threads), (size_t)lds, st,
                           static_cast<const uint16_t*>(a.X), a.qw, a.scales, a.zeros, a.zeros ? 1 : 0,
                           static_cast<uint16_t*>(a.Y), a.N, a.K, a.G, a.gshift, ks);
    }
    return hipGetLastError();
}

template <int DT>
hipError_t run_gemv8_dt(const LinearArgs& a, hipStream_t st) {
    switch (a.M) {
        case 1: return run_gemv8<DT, 1>(a, st);
        case 2: return run_gemv8<DT, 2>(a, st);
        case 3: return run_gemv8<DT, 3>(a, st);
        case 4: return run_gemv8<DT, 4>(a, st);
        case 5: return run_gemv8<DT, 5>(a, st);
        case 6: return run_gemv8<DT, 6>(a, st);
        case 7: return run_gemv8<DT, 7>(a, st);
        case 8: return run_gemv8<DT, 8>(a, st);
        case 9: return run_gemv8<DT, 9>(a, st);
        case 10: return run_gemv8<DT, 10>(a, st);
        case 11: return run_gemv8<DT, 11>(a, st);
        case 12: return run_gemv8<DT, 12>(a, st);
        case 13: return run_gemv8<DT, 13>(a, st);
        case 14: return run_gemv8<DT, 14>(a, st);
        case 15: return run_gemv8<DT, 15>(a, st);
        case 16: return run_gemv8<DT, 16>(a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool gemv8_supports(const LinearArgs& a) {
    return a.M >= 1 && a.M <= kW8MaxM && (long long)a.N * a.K < (1LL << 31) - 64;
}

hipError_t launch_gemv8(const LinearArgs& a, hipStream_t st) {
    if (!gemv8_supports(a)) return hipErrorInvalidValue;
    return a.dtype == DT_F16 ? run_gemv8_dt<DT_F16>(a, st) : run_gemv8_dt<DT_BF16>(a, st);
}

}  // namespace w4a16
