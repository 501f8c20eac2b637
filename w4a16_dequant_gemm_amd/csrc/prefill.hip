// Prefill-regime W4A16 kernel: LDS-tiled GEMM on CDNA4 matrix cores (MFMA 32x32x16).
//
// With many activation rows the layer becomes a dense contraction and compute-bound; the
// per-use dequantization then has to hide behind the matrix math (page
// "大模型推理中 Weight-only、W8A8 和 FP8 量化有什么区别？如何选型？", section 二, large-batch
// caveat; page "Quantization & Acceleration: 解释 W8A8 与 W4A16 的差异与取舍", prefill is
// compute-bound).  Weights are dequantized in registers, never written back (same page,
// section 二; page "LLM 量化中 W4A16 表示什么，它在权重位宽和激活精度上有什么取舍？",
// 性能取决于 kernel).
//
// Block tile 128 (M) x 128 (N), k-step 64, 256 threads = 4 waves in a 2x2 grid, wave
// tile 64 x 64 = 2 x 2 MFMA 32x32 tiles.
//   A operand (activations): the block stages its 128 x 64 activation tile in LDS once
//     per k-step (double-buffered), permuting each 8-column block to the unpack's pair
//     order while staging; rows are padded by 16 bytes to spread LDS banks.
//   B operand (weights): lane (n = l % 32, h = l / 32) loads 16 bytes = 32 columns
//     k0 + 32h .. k0 + 32h + 31 of weight row n; MFMA kk of the step takes word kk, i.e.
//     columns k0 + 32h + 8kk + {0,4,1,5,2,6,3,7}, and the A lane (m, h) reads the same
//     columns from LDS.  Each MFMA therefore stays inside one 64-column window, so a
//     group size that is a multiple of 64 never splits an MFMA across groups.
//   Codes: byte-permute unpack (fp16 subnormals u * 2^-24, or bf16 128 + u), so the
//     activation tile is staged in the matching "byte order".
//   Groups: the MFMAs of one group accumulate into acc_g starting from zero; at the
//     group's last step acc += s'[n] * (acc_g - c[n] * S_g[m]) with S_g the group's
//     activation sum of row m (computed while staging), fp16: s' = s * 2^24, c = z and S_g
//     in units of 2^-24; bf16: s' = s, c = 128 + z.
#include "common.h"
#include "launch.h"

namespace w4a16 {

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_STRIDE = BK + 8;   // halves per LDS row (16 B pad)

template <int DT>
struct Mfma;
template <>
struct Mfma<DT_F16> {
    static __device__ __forceinline__ f32x16 run(const uint32_t a[4], const uint32_t b[4], f32x16 c) {
        f16x8 av, bv;
        __builtin_memcpy(&av, a, 16);
        __builtin_memcpy(&bv, b, 16);
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, c, 0, 0, 0);
    }
};
template <>
struct Mfma<DT_BF16> {
    static __device__ __forceinline__ f32x16 run(const uint32_t a[4], const uint32_t b[4], f32x16 c) {
        bf16x8 av, bv;
        __builtin_memcpy(&av, a, 16);
        __builtin_memcpy(&bv, b, 16);
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, c, 0, 0, 0);
    }
};

template <int DT>
__global__ __launch_bounds__(256, 2) void prefill_kernel(const uint16_t* __restrict__ X,
                                                         const uint32_t* __restrict__ qw,
                                                         const uint16_t* __restrict__ scales,
                                                         const uint16_t* __restrict__ zeros,
                                                         int has_zeros,
                                                         uint16_t* __restrict__ Y, int M, int N,
                                                         int K, int G, int steps_per_group) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM * LDS_STRIDE];
    __shared__ float sg[2][BM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;          // wave row in the 2x2 grid
    const int wn = wave & 1;           // wave column
    const int l32 = lane & 31;
    const int h = lane >> 5;

    const int tiles_n = (N + BN - 1) / BN;
    const int tm = blockIdx.x / tiles_n;
    const int tn = blockIdx.x % tiles_n;
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int KW = K >> 3;
    const int nsteps = K / BK;

    // Staging role: thread t loads row t/2, columns 32*(t%2) .. +31 of the tile.
    // Rows past M / N are clamped to the last valid row: every load is unconditional and
    // the results of those rows are never stored.
    const int srow = tid >> 1;
    const int shalf = tid & 1;
    const uint16_t* xsrc = X + (size_t)min(m0 + srow, M - 1) * K + 32 * shalf;
    const uint16_t* zsrc = has_zeros ? zeros : scales;   // NULL zeros: value replaced by 8

    // Weight rows this lane feeds (one per n sub-tile).
    int wrow[2];
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) wrow[ns] = min(n0 + wn * 64 + ns * 32 + l32, N - 1);

    u32x4 xreg[4];
    float s_acc = 0.0f;   // running group sum of this staging row

    auto load_x = [&](int step) {
#pragma unroll
        for (int b = 0; b < 4; ++b)
            xreg[b] = *reinterpret_cast<const u32x4*>(xsrc + (size_t)step * BK + 8 * b);
    };
    auto store_x = [&](int buf, int step) {
        uint16_t* dst = &xs[buf][srow * LDS_STRIDE + 32 * shalf];
        float part = 0.0f;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            uint32_t o[4];
            permute_x8_byte(xreg[b].x, xreg[b].y, xreg[b].z, xreg[b].w, o);
            *reinterpret_cast<u32x4*>(dst + 8 * b) = u32x4{o[0], o[1], o[2], o[3]};
            part += (pair_sum<DT>(xreg[b].x) + pair_sum<DT>(xreg[b].y)) +
                    (pair_sum<DT>(xreg[b].z) + pair_sum<DT>(xreg[b].w));
        }
        part += __shfl_xor(part, 1, 64);
        s_acc += part;
        if ((step + 1) % steps_per_group == 0) {
            // fp16 codes are in units of 2^-24; scale the sum the same way (exact)
            const float sv = DT == DT_F16 ? s_acc * 5.9604644775390625e-8f : s_acc;
            if (shalf == 0) sg[(step / steps_per_group) & 1][srow] = sv;
            s_acc = 0.0f;
        }
    };

    u32x4 wreg[2];
    auto load_w = [&](int step) {
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
            wreg[ns] = *reinterpret_cast<const u32x4*>(qw + (size_t)wrow[ns] * KW +
                                                       (size_t)step * (BK / 8) + 4 * h);
    };

    f32x16 acc[2][2], accg[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    float gs[2] = {0.0f, 0.0f}, gc[2] = {0.0f, 0.0f};

    load_x(0);
    store_x(0, 0);
    load_w(0);
    __syncthreads();

    for (int step = 0; step < nsteps; ++step) {
        const int buf = step & 1;
        const int grp = step / steps_per_group;
        const bool gfirst = (step % steps_per_group) == 0;
        const bool glast = ((step + 1) % steps_per_group) == 0;
        if (gfirst) {
#pragma unroll
            for (int ns = 0; ns < 2; ++ns) {
                const float sv = h2f(scales[(size_t)wrow[ns] * G + grp]);
                const float zr = h2f(zsrc[(size_t)wrow[ns] * G + grp]);
                const float zv = has_zeros ? zr : 8.0f;
                gs[ns] = DT == DT_F16 ? sv * 16777216.0f : sv;     // fp16: fold 2^24 (exact)
                gc[ns] = DT == DT_F16 ? zv : 128.0f + zv;
            }
        }
        // Dequantize this step's weights into B operands.
        uint32_t bop[2][4][4];
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) unpack_byte<DT == DT_F16 ? 0u : 0x43u>(wreg[ns][kk], bop[ns][kk]);
        }
        // Prefetch the next step.
        if (step + 1 < nsteps) {
            load_x(step + 1);
            load_w(step + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        // MFMAs.
        const uint16_t* xb = xs[buf];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
            for (int ms = 0; ms < 2; ++ms) {
                const int r = wm * 64 + ms * 32 + l32;
                const u32x4 av = *reinterpret_cast<const u32x4*>(xb + r * LDS_STRIDE + 32 * h + 8 * kk);
                const uint32_t a[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
                for (int ns = 0; ns < 2; ++ns) {
                    if (gfirst && kk == 0) {
                        f32x16 zero;
#pragma unroll
                        for (int e = 0; e < 16; ++e) zero[e] = 0.0f;
                        accg[ms][ns] = Mfma<DT>::run(a, bop[ns][kk], zero);
                    } else {
                        accg[ms][ns] = Mfma<DT>::run(a, bop[ns][kk], accg[ms][ns]);
                    }
                }
            }
        }
        if (step + 1 < nsteps) store_x(buf ^ 1, step + 1);
        if (glast) {
#pragma unroll
            for (int ms = 0; ms < 2; ++ms) {
#pragma unroll
                for (int ns = 0; ns < 2; ++ns) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int r = wm * 64 + ms * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
                        const float v = fmaf(-gc[ns], sg[grp & 1][r], accg[ms][ns][e]);
                        acc[ms][ns][e] = fmaf(gs[ns], v, acc[ms][ns][e]);
                    }
                }
            }
        }
        __syncthreads();
    }

    // Epilogue: round to the output dtype and store.
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) {
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) {
            const int n = n0 + wn * 64 + ns * 32 + l32;
            if (n >= N) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = m0 + wm * 64 + ms * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
                if (m < M) Y[(size_t)m * N + n] = f2out<DT>(acc[ms][ns][e]);
            }
        }
    }
}

}  // namespace

bool prefill_supports(const LinearArgs& a) {
    if (a.K % BK != 0) return false;
    if (a.g % BK != 0) return false;
    return true;
}

hipError_t launch_prefill(const LinearArgs& a, hipStream_t st) {
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    const int spg = a.g / BK;
    const int hz = a.zeros ? 1 : 0;
    if (a.dtype == DT_F16)
        hipLaunchKernelGGL(prefill_kernel<DT_F16>, dim3(tiles), dim3(256), 0, st,
                           static_cast<const uint16_t*>(a.X), a.qw, a.scales, a.zeros, hz,
                           static_cast<uint16_t*>(a.Y), a.M, a.N, a.K, a.G, spg);
    else
        hipLaunchKernelGGL(prefill_kernel<DT_BF16>, dim3(tiles), dim3(256), 0, st,
                           static_cast<const uint16_t*>(a.X), a.qw, a.scales, a.zeros, hz,
                           static_cast<uint16_t*>(a.Y), a.M, a.N, a.K, a.G, spg);
    return hipGetLastError();
}

}  // namespace w4a16
