// Decode-regime W4A16 kernel: weight-streaming GEMV for small M (dot2 on the VALU).
//
// At decode the layer reads every weight once per token while doing two flops per
// weight per activation row, so it is bound by the weight stream from HBM, not by
// arithmetic (page "推理优化中“用精度换性能“的核心技术：量化", section 一; page
// "Quantization & Acceleration: 解释 W8A8 与 W4A16 的差异与取舍", decode vs prefill).
// The kernel therefore (i) reads each packed weight row exactly once with coalesced
// 128-bit loads, (ii) dequantizes in registers only (page
// "大模型推理中 Weight-only、W8A8 和 FP8 量化有什么区别？如何选型？", section 二) and
// (iii) keeps the activations resident in registers for the life of the block.
//
// Mapping.  A block of NT threads (NT a multiple of 64, <= 1024) owns RB consecutive
// output rows and the whole K range.  Thread t owns the 32-column chunks
// c = t + NT*i (i < CPL) of every row: its activation chunks (M x 32 values, permuted to
// the pair order of the unpack) are loaded once into registers, then for each row the
// thread streams one 16-byte weight chunk per owned chunk.  One 16-byte chunk (32
// columns) always lies inside one group because g is a multiple of 32, so the group's
// scale multiplies the chunk's fp32 partial sum once.  Partial sums are reduced across
// the wave with shuffles and across waves through LDS; one thread per (row, m) rounds
// to the output dtype.
#include "common.h"
#include "launch.h"

namespace w4a16 {

namespace {

// Threads per block the kernel is compiled for: configurations that hold many
// activation registers get 256 VGPRs (512 threads), the others 128 (1024 threads).
constexpr int launch_limit(int M, int CPL) { return (M * CPL <= 2 || (CPL == 1 && M <= 4)) ? 1024 : 512; }

template <int DT, int M, int CPL, int RB>
__global__ __launch_bounds__(launch_limit(M, CPL)) void gemv_kernel(const uint16_t* __restrict__ X,
                                                    const uint32_t* __restrict__ qw,
                                                    const uint16_t* __restrict__ scales,
                                                    const uint16_t* __restrict__ zeros,
                                                    uint16_t* __restrict__ Y, int N, int K, int G,
                                                    int gshift) {
    __shared__ float red[16][RB][M];
    const int tid = threadIdx.x;
    const int NT = blockDim.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nwaves = NT >> 6;
    const int C = K >> 5;
    const int KW = K >> 3;

    // Activation chunks, permuted, in registers.
    uint32_t xr[M][CPL][16];
    float xs[M][CPL];
    int cg[CPL];
    bool cval[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = tid + NT * i;
        cval[i] = c < C;
        cg[i] = group_of(c << 5, gshift);
#pragma unroll
        for (int m = 0; m < M; ++m) {
            xs[m][i] = 0.0f;
            if (cval[i]) {
                const u32x4* src = reinterpret_cast<const u32x4*>(X + (size_t)m * K + ((size_t)c << 5));
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const u32x4 v = src[b];
                    uint32_t o[4];
                    permute_x8(v.x, v.y, v.z, v.w, o);
#pragma unroll
                    for (int q = 0; q < 4; ++q) xr[m][i][4 * b + q] = o[q];
                    if constexpr (DT == DT_BF16) {
                        xs[m][i] += (pair_sum<DT>(v.x) + pair_sum<DT>(v.y)) +
                                    (pair_sum<DT>(v.z) + pair_sum<DT>(v.w));
                    }
                }
            } else {
#pragma unroll
                for (int q = 0; q < 16; ++q) xr[m][i][q] = 0u;
            }
        }
    }

    for (int row0 = blockIdx.x * RB; row0 < N; row0 += gridDim.x * RB) {
        u32x4 wv[RB][CPL];
        float sc[RB][CPL], zc[RB][CPL];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int n = row0 + r;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int c = tid + NT * i;
                if (n < N && cval[i]) {
                    wv[r][i] = *reinterpret_cast<const u32x4*>(qw + (size_t)n * KW + ((size_t)c << 2));
                    sc[r][i] = h2f(scales[(size_t)n * G + cg[i]]);
                    zc[r][i] = zeros ? h2f(zeros[(size_t)n * G + cg[i]]) : 8.0f;
                } else {
                    wv[r][i] = u32x4{0u, 0u, 0u, 0u};
                    sc[r][i] = 0.0f;
                    zc[r][i] = 0.0f;
                }
            }
        }

        float acc[RB][M];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
#pragma unroll
            for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                float part[M];
#pragma unroll
                for (int m = 0; m < M; ++m) part[m] = 0.0f;
                ZeroConst zk;
                if constexpr (DT == DT_F16) zk = make_zero_const_f16(zc[r][i]);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    uint32_t cd[4];
                    if constexpr (DT == DT_F16)
                        unpack_f16(wv[r][i][q], zk, cd);
                    else
                        unpack_bf16(wv[r][i][q], cd);
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        float p = part[m];
                        p = dot2<DT>(xr[m][i][4 * q + 0], cd[0], p);
                        p = dot2<DT>(xr[m][i][4 * q + 1], cd[1], p);
                        p = dot2<DT>(xr[m][i][4 * q + 2], cd[2], p);
                        p = dot2<DT>(xr[m][i][4 * q + 3], cd[3], p);
                        part[m] = p;
                    }
                }
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    if constexpr (DT == DT_F16) {
                        acc[r][m] = fmaf(sc[r][i], part[m], acc[r][m]);
                    } else {
                        const float corr = fmaf(-(128.0f + zc[r][i]), xs[m][i], part[m]);
                        acc[r][m] = fmaf(sc[r][i], corr, acc[r][m]);
                    }
                }
            }
        }

        // Reduce over the 64 lanes of each wave, then over the waves.
#pragma unroll
        for (int r = 0; r < RB; ++r) {
#pragma unroll
            for (int m = 0; m < M; ++m) {
                float v = acc[r][m];
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
                if (lane == 0) red[wave][r][m] = v;
            }
        }
        __syncthreads();
        if (tid < RB * M) {
            const int r = tid / M;
            const int m = tid % M;
            const int n = row0 + r;
            float v = 0.0f;
            for (int w = 0; w < nwaves; ++w) v += red[w][r][m];
            if (n < N) Y[(size_t)m * N + n] = f2out<DT>(v);
        }
        __syncthreads();
    }
}

constexpr int kRB = 4;

struct GemvCfg {
    int nt = 0;
    int cpl = 0;
};

int cpl_max(int M) { return M >= 4 ? 1 : (M == 3 ? 1 : 4 / M); }

GemvCfg pick(int M, int K) {
    const int C = K / 32;
    GemvCfg best;
    double best_util = -1.0;
    for (int cpl = 1; cpl <= cpl_max(M); ++cpl) {
        int nt = ((C + cpl - 1) / cpl + 63) / 64 * 64;
        if (nt > launch_limit(M, cpl)) continue;
        double util = (double)C / ((double)nt * cpl);
        if (util > best_util + 1e-9 || (util > best_util - 1e-9 && cpl > best.cpl)) {
            best_util = util;
            best.nt = nt;
            best.cpl = cpl;
        }
    }
    return best;
}

template <int DT, int M, int CPL>
hipError_t run(const LinearArgs& a, int nt, hipStream_t st) {
    const int blocks = (a.N + kRB - 1) / kRB;
    hipLaunchKernelGGL((gemv_kernel<DT, M, CPL, kRB>), dim3(blocks), dim3(nt), 0, st,
                       static_cast<const uint16_t*>(a.X), a.qw, a.scales, a.zeros,
                       static_cast<uint16_t*>(a.Y), a.N, a.K, a.G, a.gshift);
    return hipGetLastError();
}

template <int DT, int M>
hipError_t run_m(const LinearArgs& a, const GemvCfg& c, hipStream_t st) {
    switch (c.cpl) {
        case 1: return run<DT, M, 1>(a, c.nt, st);
        case 2: if constexpr (M <= 2) return run<DT, M, 2>(a, c.nt, st); break;
        case 3: if constexpr (M == 1) return run<DT, M, 3>(a, c.nt, st); break;
        case 4: if constexpr (M == 1) return run<DT, M, 4>(a, c.nt, st); break;
    }
    return hipErrorInvalidValue;
}

template <int DT>
hipError_t run_dt(const LinearArgs& a, const GemvCfg& c, hipStream_t st) {
    switch (a.M) {
        case 1: return run_m<DT, 1>(a, c, st);
        case 2: return run_m<DT, 2>(a, c, st);
        case 3: return run_m<DT, 3>(a, c, st);
        case 4: return run_m<DT, 4>(a, c, st);
        case 5: return run_m<DT, 5>(a, c, st);
        case 6: return run_m<DT, 6>(a, c, st);
        case 7: return run_m<DT, 7>(a, c, st);
        case 8: return run_m<DT, 8>(a, c, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool gemv_supports(const LinearArgs& a) {
    if (a.M < 1 || a.M > 8) return false;
    return pick(a.M, a.K).nt > 0;
}

hipError_t launch_gemv(const LinearArgs& a, hipStream_t st) {
    const GemvCfg c = pick(a.M, a.K);
    if (c.nt == 0) return hipErrorInvalidValue;
    return a.dtype == DT_F16 ? run_dt<DT_F16>(a, c, st) : run_dt<DT_BF16>(a, c, st);
}

}  // namespace w4a16
