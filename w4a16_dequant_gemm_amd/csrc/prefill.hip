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
#include <algorithm>

#include "common.h"
#include "launch.h"
#include "tile.h"
#include "w8.h"

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

// BITS = 8 (W8A16): 8-bit codes, four per word; lane (n, h) loads the 32 bytes holding columns
// k0 + 32h .. + 31 (two 16-byte loads), MFMA kk takes words 2kk and 2kk + 1 (columns
// k0 + 32h + 8kk .. + 7) in natural order, the activation tile is staged unpermuted, and the
// codes enter the MFMA exactly (fp16 subnormals u * 2^-24, or bf16 u), so c = z for both
// dtypes (the implicit symmetric zero point is 128).
template <int DT, int BITS = 4>
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
    const int KW = BITS == 4 ? K >> 3 : K >> 2;      // words per weight row
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
            uint32_t o[4] = {xreg[b].x, xreg[b].y, xreg[b].z, xreg[b].w};
            if constexpr (BITS == 4) permute_x8_byte(xreg[b].x, xreg[b].y, xreg[b].z, xreg[b].w, o);
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

    constexpr int WL = BITS == 4 ? 1 : 2;            // 16-byte weight loads per row and step
    u32x4 wreg[2][WL];
    auto load_w = [&](int step) {
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
#pragma unroll
            for (int i = 0; i < WL; ++i)
                wreg[ns][i] = *reinterpret_cast<const u32x4*>(qw + (size_t)wrow[ns] * KW +
                                                              (size_t)step * (BK * BITS / 32) + 4 * (WL * h + i));
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
                const float zv = has_zeros ? zr : (BITS == 4 ? 8.0f : 128.0f);
                gs[ns] = DT == DT_F16 ? sv * 16777216.0f : sv;     // fp16: fold 2^24 (exact)
                gc[ns] = (DT == DT_F16 || BITS == 8) ? zv : 128.0f + zv;
            }
        }
        // Dequantize this step's weights into B operands.
        uint32_t bop[2][4][4];
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if constexpr (BITS == 4) {
                    unpack_byte<DT == DT_F16 ? 0u : 0x43u>(wreg[ns][0][kk], bop[ns][kk]);
                } else {
                    codes8<DT>(wreg[ns][kk >> 1][2 * (kk & 1)], &bop[ns][kk][0]);
                    codes8<DT>(wreg[ns][kk >> 1][2 * (kk & 1) + 1], &bop[ns][kk][2]);
                }
            }
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

// ---------------------------------------------------------------------------------
// fp16 dequantization for the fp16 kernels that multiply dequantized weights:
// w = fp16(s * (u - z)), rounded once.
//
// The codes are fp16 subnormals u * 2^-24 taken from the packed word by masks (exact: a
// nibble in the low bits of an fp16 with a zero exponent field), in "mask order" (u0,u4)
// (16u1,16u5) (u2,u6) (16u3,16u7) for 4-bit codes.  Each weight is one mixed-precision FMA,
// fma(code, s', c) evaluated in fp32 with s' = s * 2^24 (or s * 2^20 for the x16 slots) and
// c = -s * z, its result rounded once to fp16 into the low or high half of the output
// register (v_fma_mixlo_f16 / v_fma_mixhi_f16, which read either half of a 32-bit source).
// s has 11 significant bits and u - z at most 12 (|z| <= 2048), so s' * code and the sum
// s (u - z) are exact in fp32: the single fp16 rounding is the only one, for every zero
// point the quantizers emit.  The pair (lo, hi) picks its two codes from any halves, which
// rebuilds natural column order without permutes.
template <int LO_HI, int HI_HI>
__device__ __forceinline__ uint32_t dq_pair(uint32_t src_lo, float s_lo, uint32_t src_hi, float s_hi, float c) {
    uint32_t r;
    if constexpr (LO_HI)
        asm("v_fma_mixlo_f16 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(src_lo), "v"(s_lo), "v"(c));
    else
        asm("v_fma_mixlo_f16 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(src_lo), "v"(s_lo), "v"(c));
    if constexpr (HI_HI)
        asm("v_fma_mixhi_f16 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(r) : "v"(src_hi), "v"(s_hi), "v"(c));
    else
        asm("v_fma_mixhi_f16 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "+v"(r) : "v"(src_hi), "v"(s_hi), "v"(c));
    return r;
}

// The fp32 constants of one (row, group): s * 2^24, s * 2^20 and -s * z (all exact).
struct DqConst {
    float s24, s20, c;
};
__device__ __forceinline__ DqConst dq_const(uint16_t s_bits, float z) {
    const float s = h2f(s_bits);
    return DqConst{s * 16777216.0f, s * 1048576.0f, -s * z};
}

// One packed word of 4-bit codes (8 consecutive columns) -> four fp16 pairs in natural order.
__device__ __forceinline__ void dq_word4(uint32_t w, const DqConst& q, uint32_t out[4]) {
    const uint32_t w8 = w >> 8;
    const uint32_t m0 = w & 0x000F000Fu;     // u0 u4
    const uint32_t m1 = w & 0x00F000F0u;     // 16 u1, 16 u5
    const uint32_t m2 = w8 & 0x000F000Fu;    // u2 u6
    const uint32_t m3 = w8 & 0x00F000F0u;    // 16 u3, 16 u7
    out[0] = dq_pair<0, 0>(m0, q.s24, m1, q.s20, q.c);    // (u0, u1)
    out[1] = dq_pair<0, 0>(m2, q.s24, m3, q.s20, q.c);    // (u2, u3)
    out[2] = dq_pair<1, 1>(m0, q.s24, m1, q.s20, q.c);    // (u4, u5)
    out[3] = dq_pair<1, 1>(m2, q.s24, m3, q.s20, q.c);    // (u6, u7)
}

// One 32-bit word of 8-bit codes (4 consecutive columns) -> two fp16 pairs in natural order.
__device__ __forceinline__ void dq_word8(uint32_t w, const DqConst& q, uint32_t out[2]) {
    const uint32_t p0 = perm(0u, w, 0x0C010C00u);          // (u0, u1) as subnormals
    const uint32_t p1 = perm(0u, w, 0x0C030C02u);          // (u2, u3)
    out[0] = dq_pair<0, 1>(p0, q.s24, p0, q.s24, q.c);
    out[1] = dq_pair<0, 1>(p1, q.s24, p1, q.s24, q.c);
}

// ---------------------------------------------------------------------------------
// fp16 kernel: dequantize once per block into LDS.
//
// Block tile 256 (M) x 128 (N), k-step 32, 256 threads = 4 waves in a 2 x 2 grid, wave
// tile 128 x 64 = 4 x 2 MFMA 32x32x16 tiles.  Per k-step every thread
//   - loads 64 bytes of one activation row (its 32 columns) and stores them to LDS
//     unchanged (natural column order),
//   - loads 8 bytes = 16 codes of one weight row and writes the dequantized fp16 weights
//     fp16(s * (u - z)) to LDS (dq_word4: masks and one mixed-precision FMA per weight,
//     one rounding),
// so every weight is dequantized exactly once per block -- the pages' "dequantize the
// INT4 weight to FP16, then multiply" with the FP16 weight living only in LDS.  The
// MFMAs read both operands from LDS in natural order; rows are padded by 16 bytes,
// which makes the 32-lane column reads conflict-free.  LDS is double-buffered, one
// barrier per k-step.
constexpr int F_BM = 256, F_BN = 128, F_BK = 32;
constexpr int F_LDA = F_BK + 8;      // halves per LDS row

__global__ __launch_bounds__(256, 2) void prefill_f16_kernel(
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int has_zeros,
    uint16_t* __restrict__ Y, int M, int N, int K, int G, int gshift) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][F_BM * F_LDA];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][F_BN * F_LDA];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int l32 = lane & 31;
    const int h = lane >> 5;
    const int tiles_n = (N + F_BN - 1) / F_BN;
    const int m0 = (blockIdx.x / tiles_n) * F_BM;
    const int n0 = (blockIdx.x % tiles_n) * F_BN;
    const int KW = K >> 3;
    const int nsteps = K / F_BK;

    // Staging roles.  Activations: thread t owns row t of the tile.  Weights: thread t
    // owns row t/2, columns 16*(t%2) .. +15 of the step (two words).  Rows past M / N are
    // clamped (loads stay in bounds; their results are never stored).
    const uint16_t* xrow = X + (size_t)min(m0 + tid, M - 1) * K;
    const int wr = tid >> 1;
    const int wh = tid & 1;
    const int wrow = min(n0 + wr, N - 1);
    const uint32_t* wsrc = qw + (size_t)wrow * KW + 2 * wh;
    const uint16_t* zsrc = has_zeros ? zeros : scales;    // NULL zeros: value replaced by 8

    u32x4 xa[4];
    uint32_t wq[2];
    auto load_step = [&](int step) {
#pragma unroll
        for (int b = 0; b < 4; ++b)
            xa[b] = *reinterpret_cast<const u32x4*>(xrow + (size_t)step * F_BK + 8 * b);
        const uint2 v = *reinterpret_cast<const uint2*>(wsrc + (size_t)step * (F_BK / 8));
        wq[0] = v.x;
        wq[1] = v.y;
    };
    // dequantization constants of the current group
    DqConst dq{0.0f, 0.0f, 0.0f};
    int cur_group = -1;
    auto store_step = [&](int buf, int step) {
        const int grp = group_of(step * F_BK, gshift);
        if (grp != cur_group) {
            cur_group = grp;
            dq = dq_const(scales[(size_t)wrow * G + grp], has_zeros ? h2f(zsrc[(size_t)wrow * G + grp]) : 8.0f);
        }
        uint16_t* arow = &As[buf][tid * F_LDA];
#pragma unroll
        for (int b = 0; b < 4; ++b) *reinterpret_cast<u32x4*>(arow + 8 * b) = xa[b];
        uint32_t d[8];
        dq_word4(wq[0], dq, &d[0]);
        dq_word4(wq[1], dq, &d[4]);
        uint16_t* brow = &Bs[buf][wr * F_LDA + 16 * wh];
        *reinterpret_cast<u32x4*>(brow) = u32x4{d[0], d[1], d[2], d[3]};
        *reinterpret_cast<u32x4*>(brow + 8) = u32x4{d[4], d[5], d[6], d[7]};
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    load_step(0);
    store_step(0, 0);
    __syncthreads();
    for (int step = 0; step < nsteps; ++step) {
        const int buf = step & 1;
        if (step + 1 < nsteps) load_step(step + 1);
        const uint16_t* A = As[buf];
        const uint16_t* B = Bs[buf];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            uint32_t bf[2][4];
#pragma unroll
            for (int ns = 0; ns < 2; ++ns) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(
                    B + (wn * 64 + ns * 32 + l32) * F_LDA + 16 * ks + 8 * h);
                bf[ns][0] = v.x; bf[ns][1] = v.y; bf[ns][2] = v.z; bf[ns][3] = v.w;
            }
#pragma unroll
            for (int ms = 0; ms < 4; ++ms) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(
                    A + (wm * 128 + ms * 32 + l32) * F_LDA + 16 * ks + 8 * h);
                const uint32_t af[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int ns = 0; ns < 2; ++ns) acc[ms][ns] = Mfma<DT_F16>::run(af, bf[ns], acc[ms][ns]);
            }
        }
        if (step + 1 < nsteps) store_step(buf ^ 1, step + 1);
        __syncthreads();
    }

#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) {
            const int n = n0 + wn * 64 + ns * 32 + l32;
            if (n >= N) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = m0 + wm * 128 + ms * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
                if (m < M) Y[(size_t)m * N + n] = f2h_bits(acc[ms][ns][e]);
            }
        }
    }
}

// ---------------------------------------------------------------------------------
// fp16 kernel, wide variant (K % 128 == 0): block tile 256 (M) x 256 (N), k-step 64,
// 4 waves side by side along N, wave tile 256 x 64 = 8 x 2 MFMA 32x32x16 tiles.
//   Activations: the block's 256 x 64 tile goes global -> LDS directly (16-byte buffer
//     loads with the LDS destination: lane l of an instruction writes slot base + l), two
//     buffers.  Row r is 8 slots of 16 bytes; column piece c of row r sits in slot
//     c ^ ((r / 2) % 8), which keeps the 32-row fragment reads free of bank conflicts.
//     Every wave reads all 256 rows; the LDS carries only activations.
//   Weights: each wave dequantizes exactly the 64 weight rows it multiplies, in
//     registers (none goes through LDS, none is dequantized twice): lane (n, h) loads the
//     16 bytes holding columns 32 h .. 32 h + 31 of the step for each of its two rows, one
//     step ahead, and turns word j into the fp16 B fragment of MFMA j (dq_word4: one
//     mixed-precision FMA per weight, exact in fp32, one rounding to fp16).  MFMA j covers columns 8 j .. 8 j + 7 and 32 + 8 j .. + 7; the activation
//     fragment of lane (m, h) reads the same columns.  The next step's dequantization is
//     interleaved with this step's MFMAs.
//   Block order: consecutive block indices run on different XCDs; blocks are renumbered
//     so that each XCD works through consecutive tiles (a few 256-row activation panels,
//     held in that XCD's L2).
// Device-only builtins behind device functions: inside a lambda whose body depends on a
// kernel template parameter, a raw builtin makes the host pass drop the kernel's launch stub.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, u32x4* dst, int voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
}
template <int MASK, int N>
__device__ __forceinline__ void sched_group() {
    __builtin_amdgcn_sched_group_barrier(MASK, N, 0);
}
// Wait until at most N vector-memory loads of this wave are in flight.  Written as an asm
// statement with a memory clobber, it is also a compiler barrier: no load moves across it,
// so N counts exactly the loads issued after the ones waited for.
template <int N>
struct VmWait {
    static constexpr int value = N;
};
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"I"(N) : "memory");
}
// Keeps the loads before it ahead of the loads after it in issue order.
__device__ __forceinline__ void issue_fence() { asm volatile("" ::: "memory"); }

constexpr int W_BM = 256, W_BN = 256, W_BK = 64;     // K % 128 == 0: steps in pairs

// BITS = 8 (W8A16): lane (n, h) loads the 32 bytes of columns 32h .. 32h + 31 (two 16-byte
// loads) and MFMA j takes words 2j and 2j + 1 (one byte permute per pair instead of the nibble
// masks (dq_word8), the implicit symmetric zero point is 128).
// Split K (part != NULL): block (x, y) runs k-steps [y * spl, (y + 1) * spl) of its tile and
// stores the fp32 partial tile to part[y][M][N]; splitk_reduce_kernel sums the partials in
// split order.  Without a split, spl = K / 64, grid y = 1 and the tile goes to Y.
//
// KG = 2 splits K inside the block: wave w works on columns 64 (w % 4) ... of the tile over the
// k-steps of parity w / 4 (two wave groups in lockstep, each with its own activation tiles),
// and the second group's accumulators are added to the first's through LDS at the end, in
// fixed order.  It doubles the waves per SIMD for tiles of 64 and 128 rows, which a grid of at
// most one block per CU otherwise runs one wave per SIMD, without any buffer outside the block.
// The host launches KG = 2 only when each group's step count is even (K % 256 == 0), which the
// two-step loop needs; with KG = 2 the 64-row tile runs that loop, not the three-step one.
//
// SZL: the block's scales and zeros for its k-range sit in LDS (dynamic, gp dwords per weight
// row, s | z << 16, gp odd so the 32 rows a wave reads per step fall in distinct banks),
// staged once at the start by one thread per row with 16-byte loads.  Loading them per step
// instead costs four 2-byte loads per wave and step, each touching 32 rows' cache lines: with
// 64-row tiles that was half of the address unit's work, and the address unit, not the
// matrix cores, set the pace.
template <bool HZ, int BITS = 4, bool SPLIT = false, int MS = 8, int KG = 1, bool SZL = false, bool PH = false>
__global__ __launch_bounds__(256 * KG, (MS >= 8 || BITS == 8 || (MS == 2 && !SPLIT) || KG > 1 || SZL) ? 1 : 2) void prefill_f16_wide_kernel(
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros,
    uint16_t* __restrict__ Y, int M, int N, int K, int G, int gshift,
    float* __restrict__ part = nullptr, int spl = 0, int gp = 0, int pst = 0) {
    static_assert(KG == 1 || (KG == 2 && BITS == 4 && !SPLIT && MS <= 4), "k-groups: 4-bit, plain, <= 128 rows");
    static_assert(!PH || (SZL && !SPLIT), "phases: staged scales and zeros, plain launch");
    constexpr int BMk = 32 * MS;                                       // block rows
    constexpr int ASZ = BMk * 8;                                       // one group's tile, 16-byte slots
    // the activation double buffer as two LDS objects, so that the compiler's wait before a
    // fragment read covers only the loads into that buffer (one object would make every read
    // wait for the other buffer's loads, issued for the next step)
    __shared__ __attribute__((aligned(16))) u32x4 As0[KG * ASZ];       // 32 KB at 256 rows
    __shared__ __attribute__((aligned(16))) u32x4 As1[KG * ASZ];
    // 64-row blocks with one wave group run three steps deep (below): a third activation buffer
    constexpr bool DEEP = MS == 2 && BITS == 4 && !SPLIT && KG == 1;
    __shared__ __attribute__((aligned(16))) u32x4 As2[DEEP ? KG * ASZ : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = (tid >> 6) & 3;                     // column quarter of the tile
    const int kg = KG > 1 ? tid >> 8 : 0;                 // k-step parity of this wave's group
    const int abase = kg * ASZ;                           // this group's activation tiles
    const int l32 = lane & 31;
    const int h = lane >> 5;
    int mt, nt;
    if (!xcd_tile(blockIdx.x, (M + BMk - 1) / BMk, (N + W_BN - 1) / W_BN, mt, nt)) return;
    const int m0 = mt * BMk;
    const int n0 = nt * W_BN;
    const int nsteps = K / W_BK;
    const int sb = SPLIT ? blockIdx.y * spl : 0;          // this block's k-steps [sb, se), even count
    const int se = SPLIT ? min(nsteps, sb + spl) : nsteps;
    if constexpr (SPLIT) {
        if (sb >= se) return;                             // never planned (every split has steps)
    }
    // The k-range runs in phases [pb, pe) of pst k-steps each (PH; else one phase), every phase
    // with its own staged scales and zeros (SZL) and its own pipeline fill.  Local step t
    // of this group is k-step pb + kg + KG t; L local steps per group and phase; a load past the
    // group's last step re-reads that step (unused).
    int pb = sb;
    int pe = PH ? min(se, sb + pst) : se;
    int L = (pe - pb) / KG;
    auto gstep = [&](int t) { return pb + kg + KG * min(t, L - 1); };
    // SZL: groups [g0, g0 + gl) of the phase, staged in LDS
    extern __shared__ __attribute__((aligned(16))) uint32_t szl[];
    int g0 = SZL ? (pb * W_BK) >> gshift : 0;
    int gl = SZL ? (((pe * W_BK) - 1) >> gshift) + 1 - g0 : 0;

    // Buffer loads: per-lane 32-bit offsets fixed for the whole K loop, the step's offset
    // as the wave-uniform soffset.  Rows past M / N are clamped (loaded, never stored).
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(X), 0, 0x7FFFFFFF, 0x00020000);
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(qw), 0, 0x7FFFFFFF, 0x00020000);
    const uint16_t* zsrc = HZ ? zeros : scales;           // NULL zeros: value replaced by 8
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(scales), 0, 0x7FFFFFFF, 0x00020000);
    const __amdgpu_buffer_rsrc_t rz =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(zsrc), 0, 0x7FFFFFFF, 0x00020000);

    // activation staging: instruction j of wave w fills slots (MS w + j) * 64 + lane, i.e.
    // row r = (MS w + j) * 8 + lane / 8, slot lane % 8, which holds column piece
    // (lane % 8) ^ ((r / 2) % 8)
    int xoff[MS];
#pragma unroll
    for (int j = 0; j < MS; ++j) {
        const int r = (MS * wave + j) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        xoff[j] = (min(m0 + r, M - 1) * K + 8 * c) * 2;
    }
    int woff[2], szoff[2];
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) {
        const int wrow = min(n0 + 64 * wave + 32 * ns + l32, N - 1);
        woff[ns] = wrow * (BITS == 4 ? K / 2 : K) + (BITS == 4 ? 16 : 32) * h;
        szoff[ns] = wrow * G * 2;
    }
    auto load_a = [&](u32x4* As, int step) {
        // the step offset is wave-uniform; saying so keeps it in an SGPR (held in a VGPR, the
        // compiler wrapped each load in a waterfall loop)
        const int so = __builtin_amdgcn_readfirstlane(step * W_BK * 2);
#pragma unroll
        for (int j = 0; j < MS; ++j) lds_load16(rx, &As[abase + (MS * wave + j) * 64], xoff[j], so);
    };
    constexpr int WL = BITS == 4 ? 1 : 2;        // 16-byte weight loads per row and step
    struct WStage {
        u32x4 w[2][WL];
        uint16_t s[2], z[2];
    };
    auto load_w = [&](WStage& st, int step) {
        const int grp = group_of(step * W_BK + 32 * h, gshift);
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) {
#pragma unroll
            for (int i = 0; i < WL; ++i)
                st.w[ns][i] = __builtin_amdgcn_raw_buffer_load_b128(rw, woff[ns] + 16 * i, step * (W_BK / 8 * BITS), 0);
            if constexpr (SZL) {
                const uint32_t v = szl[(64 * wave + 32 * ns + l32) * gp + grp - g0];
                st.s[ns] = (uint16_t)v;
                st.z[ns] = (uint16_t)(v >> 16);
            } else {
                st.s[ns] = __builtin_amdgcn_raw_buffer_load_b16(rs, szoff[ns] + grp * 2, 0, 0);
                st.z[ns] = __builtin_amdgcn_raw_buffer_load_b16(rz, szoff[ns] + grp * 2, 0, 0);
            }
        }
    };
    // dequantization constants of a stage's two rows (per row and group)
    struct WConst {
        DqConst q[2];
    };
    auto stage_const = [&](const WStage& st) {
        WConst c;
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
            c.q[ns] = dq_const(st.s[ns], HZ ? h2f(st.z[ns]) : (BITS == 4 ? 8.0f : 128.0f));
        return c;
    };
    // word j of both rows of a stage -> the fp16 B fragments of MFMA j: b[ns][j][4]
    auto dequant_word = [&](const WStage& st, const WConst& wc, int j, uint32_t b[2][4][4]) {
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) {
            if constexpr (BITS == 4) {
                dq_word4(st.w[ns][0][j], wc.q[ns], b[ns][j]);
            } else {
                dq_word8(st.w[ns][j >> 1][2 * (j & 1)], wc.q[ns], &b[ns][j][0]);       // columns 0..3
                dq_word8(st.w[ns][j >> 1][2 * (j & 1) + 1], wc.q[ns], &b[ns][j][2]);   // columns 4..7
            }
        }
    };

    f32x16 acc[MS][2];
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // fragment slots: row m = 32 ms + l32, piece c = 4 h + j -> slot m * 8 + (c ^ (m / 2 % 8))
    int fslot[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) fslot[j] = l32 * 8 + ((4 * h + j) ^ ((l32 >> 1) & 7));

    // One step: MFMAs on the activations in LDS buffer `buf` and the dequantized weights
    // `bc`, while the next step's packed weights `nx` are dequantized into `bn`, one word
    // per MFMA group so the VALU work hides under the matrix instructions.
    auto compute = [&](const u32x4* A, const uint32_t bc[2][4][4], const WStage& nx, uint32_t bn[2][4][4]) {
        const WConst nc = stage_const(nx);
        u32x4 fa[MS], fb[MS];      // activation fragments one MFMA group ahead
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) fa[ms] = A[ms * 256 + fslot[0]];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x4* cur = (j & 1) ? fb : fa;
            u32x4* nxt = (j & 1) ? fa : fb;
            if (j < 3) {
#pragma unroll
                for (int ms = 0; ms < MS; ++ms) nxt[ms] = A[ms * 256 + fslot[j + 1]];
            }
#pragma unroll
            for (int ms = 0; ms < MS; ++ms) {
                const uint32_t af[4] = {cur[ms].x, cur[ms].y, cur[ms].z, cur[ms].w};
#pragma unroll
                for (int ns = 0; ns < 2; ++ns) acc[ms][ns] = Mfma<DT_F16>::run(af, bc[ns][j], acc[ms][ns]);
            }
            dequant_word(nx, nc, j, bn);
            // interleave: one fragment read and a few dequant instructions per MFMA pair
#pragma unroll
            for (int i = 0; i < MS; ++i) {
                if (j < 3) sched_group<0x100, 1>();   // DS read
                sched_group<0x008, 1>();              // MFMA
                sched_group<0x002, 5>();              // VALU
                sched_group<0x008, 1>();              // MFMA
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Pipeline: activations one step ahead (global -> LDS), packed weights two steps ahead
    // and dequantized weights one step ahead (registers).  A step issues the next step's
    // activation loads and the packed weights of the step after, and ends once the next
    // activation tile is in LDS (step_end), leaving the weight loads in flight: they are needed
    // one step later.  Loads past the last step re-read it (harmless, unused).
    // End of a step: this wave's loads into the next activation buffer must have landed
    // before the barrier (other waves read them after it).  The wait is explicit: each step
    // issues its activation loads (MS), a fence, then its weight loads (NWL), so the number
    // of loads allowed in flight is exact (W: the loads issued after the tile waited for);
    // the bare s_barrier leaves those weight loads in flight.  (Leaving the wait to the
    // compiler's tracking of loads into LDS failed where it issued the activation loads in a
    // waterfall loop and rotated the k-loop: one step end of the three-step pipeline carried
    // no wait at all, and a step now and then computed on the previous activation tile.)
    constexpr int NWL = 2 * (WL + (SZL ? 0 : 2));     // loads of one load_w
    auto step_end = [&](auto w) {
        wait_vmcnt<decltype(w)::value>();
        __builtin_amdgcn_s_barrier();
    };
    using After1 = VmWait<NWL>;                       // tile issued this step: its weight loads
    using After2 = VmWait<MS + 2 * NWL>;              // tile issued a step earlier (three-step)
    for (;;) {                                            // phases
    if constexpr (SZL) {
        const __amdgpu_buffer_rsrc_t rnull =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(scales), 0, 0, 0x00020000);
        stage_sz_rows<KG>(szl, gp, tid, W_BN, n0, N, G, g0, gl, HZ, rs, rz, rnull);
        __syncthreads();
    }
    if constexpr (DEEP) {
        // 64-row blocks: a k-step's matrix work (16 MFMAs per wave) is shorter than a memory
        // round trip, so with one step of prefetch every step waited for its loads (1.2 us per
        // step against about 0.45 us of MFMA).  Three stages: step s computes on activation
        // buffer s % 3 and dequantized weights b[s % 3], dequantizes packed stage (s + 1) % 3,
        // and issues the activations of step s + 2 and the packed weights of step s + 3 (into
        // the stage step s's weights left); it ends once the activations of step s + 1 are in.
        WStage p0, p1, p2;
        uint32_t b0[2][4][4], b1[2][4][4], b2[2][4][4];
        load_a(As0, gstep(0));
        load_a(As1, gstep(1));
        load_w(p0, gstep(0));
        load_w(p1, gstep(1));
        load_w(p2, gstep(2));
#pragma unroll
        for (int j = 0; j < 4; ++j) dequant_word(p0, stage_const(p0), j, b0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        // the loop body is one basic block: with a branch between its steps the compiler sank
        // each weight load into the block of its use, undoing the prefetch
        int t = 0;
        for (; t + 3 <= L; t += 3) {
            load_a(As2, gstep(t + 2));
            issue_fence();
            load_w(p0, gstep(t + 3));
            compute(As0 + abase, b0, p1, b1);
            step_end(After2{});                           // As1
            load_a(As0, gstep(t + 3));
            issue_fence();
            load_w(p1, gstep(t + 4));
            compute(As1 + abase, b1, p2, b2);
            step_end(After2{});                           // As2
            load_a(As1, gstep(t + 4));
            issue_fence();
            load_w(p2, gstep(t + 5));
            compute(As2 + abase, b2, p0, b0);
            step_end(After2{});                           // As0
        }
        // the last one or two steps: their activations and weights are already in flight
        if (t < L) {                                      // uniform
            compute(As0 + abase, b0, p1, b1);
            step_end(VmWait<0>{});                        // As1, the last tile issued
            if (t + 1 < L) compute(As1 + abase, b1, p2, b2);
        }
    } else {
        WStage p0, p1;
        uint32_t b0[2][4][4], b1[2][4][4];
        load_a(As0, gstep(0));
        load_w(p0, gstep(0));
        load_w(p1, gstep(1));
#pragma unroll
        for (int j = 0; j < 4; ++j) dequant_word(p0, stage_const(p0), j, b0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        for (int t = 0; t < L; t += 2) {
            load_a(As1, gstep(t + 1));
            issue_fence();
            load_w(p0, gstep(t + 2));
            compute(As0 + abase, b0, p1, b1);
            step_end(After1{});                           // As1
            load_a(As0, gstep(t + 2));
            issue_fence();
            load_w(p1, gstep(t + 3));
            compute(As1 + abase, b1, p0, b0);
            step_end(After1{});                           // As0
        }
    }
    if (!PH || pe >= se) break;                           // uniform
    // next phase: every load of this one has landed (the last steps' prefetches re-read into
    // the buffers the next fill writes) and every wave is done with its staged words
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    pb = pe;
    pe = min(se, pb + pst);
    L = (pe - pb) / KG;
    g0 = (pb * W_BK) >> gshift;
    gl = (((pe * W_BK) - 1) >> gshift) + 1 - g0;
    }

    if constexpr (KG > 1) {
        // group 1's accumulators into group 0's, one 32-row tile at a time through the activation
        // buffers (free once every load into them has landed): 8 KB per wave and round
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        constexpr int R0 = KG * ASZ / 512;                // 8 KB regions in As0
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
            __syncthreads();
            float* red = reinterpret_cast<float*>(wave < R0 ? As0 + wave * 512 : As1 + (wave - R0) * 512);
            if (kg == 1) {
#pragma unroll
                for (int ns = 0; ns < 2; ++ns)
#pragma unroll
                    for (int e = 0; e < 16; ++e) red[(ns * 16 + e) * 64 + lane] = acc[ms][ns][e];
            }
            __syncthreads();
            if (kg == 0) {
#pragma unroll
                for (int ns = 0; ns < 2; ++ns)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[ms][ns][e] += red[(ns * 16 + e) * 64 + lane];
            }
        }
        if (kg == 1) return;
    }

#pragma unroll
    for (int ms = 0; ms < MS; ++ms) {
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) {
            const int n = n0 + 64 * wave + 32 * ns + l32;
            if (n >= N) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = m0 + 32 * ms + 8 * (e >> 2) + 4 * h + (e & 3);
                if (m < M) {
                    if constexpr (SPLIT)
                        part[((size_t)blockIdx.y * M + m) * N + n] = acc[ms][ns][e];
                    else
                        Y[(size_t)m * N + n] = f2h_bits(acc[ms][ns][e]);
                }
            }
        }
    }
}

// Y = fp16(sum over the S splits of part[s]), in split order (deterministic).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int S,
                                                            long long MN, uint16_t* __restrict__ Y) {
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < MN; i += (long long)gridDim.x * 256) {
        float v = part[i];
        for (int sp = 1; sp < S; ++sp) v += part[(size_t)sp * MN + i];
        Y[i] = f2h_bits(v);
    }
}

}  // namespace

constexpr int kLdsPerCu = 160 * 1024;

// One launch of an instantiation of the wide kernel.  SZL kernels take 256 * gp * 4 bytes of
// dynamic LDS next to their static activation buffers; the per-kernel limit on dynamic LDS
// (64 KB by default) is raised on every launch.
template <bool HZ, int BITS, bool SPLIT, int MS, int KG, bool SZL, bool PH = false>
hipError_t launch_wide_k(dim3 grid, const LinearArgs& a, float* part, int spl, int gp, hipStream_t st,
                         int pst = 0) {
    const int dyn = SZL ? 256 * gp * 4 : 0;
    if constexpr (SZL) {
        const hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&prefill_f16_wide_kernel<HZ, BITS, SPLIT, MS, KG, SZL, PH>),
            hipFuncAttributeMaxDynamicSharedMemorySize, dyn);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((prefill_f16_wide_kernel<HZ, BITS, SPLIT, MS, KG, SZL, PH>), grid, dim3(256 * KG), dyn, st,
                       static_cast<const uint16_t*>(a.X), a.qw, a.scales, a.zeros, static_cast<uint16_t*>(a.Y),
                       a.M, a.N, a.K, a.G, a.gshift, part, spl, gp, pst);
    return hipGetLastError();
}

// LDS staging of a wide-kernel launch's scales and zeros: gp, the row stride (dwords, odd), or
// 0 when they are loaded per step; pst, the phase length in k-steps, or 0 for one phase.  The
// groups of a phase must number at most 8 kSzStagePieces and fit the LDS next to the
// activation buffers.  One phase covers a block's whole k-range (all of K, or the largest
// split); a plain launch whose rows hold more groups runs phases that start on group
// boundaries, of a multiple of 2 KG steps (the pipeline's step pairs), as few as fit.
// Measured (fp16, g = 64, 172 groups per row, 11008 -> 4096; two phases against per-step
// loads): M = 256: 158.1 -> 112.7 us, M = 1024: 163.3 -> 125.0 us, M = 2048: 218.3 -> 186.2 us,
// M = 4096: 333.1 -> 313.5 us.
struct SzlPlan {
    int gp = 0, pst = 0;
};
SzlPlan wide_szl_plan(const LinearArgs& a, int ms, int kg, bool split, int spl) {
    const int nsteps = a.K / W_BK;
    const bool deep = ms == 2 && !split && kg == 1;
    const int stat = kg * 4096 * ms * (deep ? 3 : 2);
    auto fits = [&](int gl) { return gl <= 8 * kSzStagePieces && stat + 256 * (gl | 1) * 4 <= kLdsPerCu; };
    int gl = 0;
    for (int sb = 0; sb < nsteps; sb += split ? spl : nsteps) {
        const int se = split ? std::min(nsteps, sb + spl) : nsteps;
        gl = std::max(gl, (((se * W_BK) - 1) >> a.gshift) + 1 - ((sb * W_BK) >> a.gshift));
    }
    SzlPlan p;
    if (fits(gl)) {
        p.gp = gl | 1;
        return p;
    }
    if (split) return p;
    const int q = std::max(2 * kg, a.g > W_BK ? a.g / W_BK : 1);      // steps: a multiple of q
    for (int np = 2; np <= 16; ++np) {
        const int pst = ((nsteps + np - 1) / np + q - 1) / q * q;
        if (pst >= nsteps) continue;
        const int glp = (((pst * W_BK) - 1) >> a.gshift) + 1;          // phases start on a group
        if (fits(glp)) {
            p.gp = glp | 1;
            p.pst = pst;
            return p;
        }
    }
    return p;
}


// Split-K plan of the 256 x 256 fp16 kernel for a problem with fewer tiles than CUs: splits of
// spl k-steps (even, >= 16), S = ceil(steps / spl) of them, so every split is non-empty and
// S * tiles stays near 256.  S <= 1 means no split.
void splitk_plan(const LinearArgs& a, int& S, int& spl) {
    S = 1;
    spl = a.K / W_BK;
    if (a.dtype != DT_F16 || a.K % (2 * W_BK) != 0 || a.M <= 32) return;
    if (!((long long)a.M * a.K * 2 < (1LL << 31) && (long long)a.N * (a.K / 2) < (1LL << 31) &&
          (long long)a.N * a.G * 2 < (1LL << 31)))
        return;
    const long long tiles = (long long)((a.M + W_BM - 1) / W_BM) * ((a.N + W_BN - 1) / W_BN);
    if (tiles >= 128) return;
    const int nsteps = a.K / W_BK;
    const int want = (int)(256 / tiles);
    int l = (nsteps + want - 1) / want;
    l = l < 16 ? 16 : l + (l & 1);
    S = (nsteps + l - 1) / l;
    spl = l;
}

int prefill_splitk_splits(const LinearArgs& a) {
    int S, spl;
    splitk_plan(a, S, spl);
    return S;
}

long long prefill_splitk_bytes(const LinearArgs& a) {
    const int S = prefill_splitk_splits(a);
    return S > 1 ? (long long)S * a.M * a.N * 4 : 0;
}

hipError_t launch_prefill_splitk(const LinearArgs& a, float* work, hipStream_t st) {
    int S, spl;
    splitk_plan(a, S, spl);
    if (S <= 1 || !work) return hipErrorInvalidValue;
    const int tiles = ((a.M + W_BM - 1) / W_BM) * ((a.N + W_BN - 1) / W_BN);
    const dim3 grid(8 * ((tiles + 7) / 8), S);
    const int gp = wide_szl_plan(a, 8, 1, true, spl).gp;
    hipError_t e;
    if (a.zeros)
        e = gp > 0 ? launch_wide_k<true, 4, true, 8, 1, true>(grid, a, work, spl, gp, st)
                   : launch_wide_k<true, 4, true, 8, 1, false>(grid, a, work, spl, 0, st);
    else
        e = gp > 0 ? launch_wide_k<false, 4, true, 8, 1, true>(grid, a, work, spl, gp, st)
                   : launch_wide_k<false, 4, true, 8, 1, false>(grid, a, work, spl, 0, st);
    if (e != hipSuccess) return e;
    const long long MN = (long long)a.M * a.N;
    const long long blocks = (MN + 255) / 256;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, st,
                       work, S, MN, static_cast<uint16_t*>(a.Y));
    return hipGetLastError();
}

// Rows per block of the wide kernel (MS 32-row MFMA tiles): 256, halved while the grid has
// fewer than 160 blocks and the halved tile still gives at most one block per CU (a smaller
// tile dequantizes the same weights for fewer rows, so it only pays where CUs would idle).
// Measured (plain call, g = 128): M = 256, 4096 -> 11008: 104.8 -> 76.8 us (64 rows);
// M = 1024, 11008 -> 4096: 272 -> 203 us (64 rows); M = 2048, 11008 -> 4096: 282 -> 245 us
// (128 rows); M = 1024, 4096 -> 11008 keeps 256 rows (172 blocks: 125 us, 138 us at 128).
int wide_blocks(int M, int N, int ms) { return ((M + 32 * ms - 1) / (32 * ms)) * ((N + W_BN - 1) / W_BN); }
int wide_ms(int M, int N) {
    int ms = 8;
    while (ms > 2 && (long long)wide_blocks(M, N, ms) < 160 && (long long)wide_blocks(M, N, ms / 2) <= 256) ms /= 2;
    return ms;
}

template <bool HZ, int BITS, int MS, int KG>
hipError_t launch_wide_ms(dim3 grid, const LinearArgs& a, const SzlPlan& sp, hipStream_t st) {
    if (sp.gp > 0 && sp.pst > 0)
        return launch_wide_k<HZ, BITS, false, MS, KG, true, true>(grid, a, nullptr, 0, sp.gp, st, sp.pst);
    if (sp.gp > 0) return launch_wide_k<HZ, BITS, false, MS, KG, true>(grid, a, nullptr, 0, sp.gp, st);
    return launch_wide_k<HZ, BITS, false, MS, KG, false>(grid, a, nullptr, 0, 0, st);
}

template <bool HZ, int BITS>
hipError_t launch_wide(const LinearArgs& a, hipStream_t st) {
    const int ms = wide_ms(a.M, a.N);
    // 64- and 128-row tiles (grids of at most one block per CU) split K over two wave groups
    // when the step count allows: two waves per SIMD issue VALU work twice as fast as one.
    // Measured (fp16, g = 128, scales and zeros in LDS): M = 256, 4096 -> 11008: 54.9 -> 49.2 us;
    // M = 1024, 11008 -> 4096: 152.0 -> 139.1 us; M = 2048, 11008 -> 4096: 205.7 -> 196.6 us.
    const int kg = BITS == 4 && ms <= 4 && (a.K / W_BK) % 4 == 0 ? 2 : 1;
    const SzlPlan sp = wide_szl_plan(a, ms, kg, false, 0);
    const int tiles = wide_blocks(a.M, a.N, ms);
    const dim3 grid(8 * ((tiles + 7) / 8));
    if constexpr (BITS == 4) {
        if (kg == 2) {
            if (ms == 4) return launch_wide_ms<HZ, 4, 4, 2>(grid, a, sp, st);
            if (ms == 2) return launch_wide_ms<HZ, 4, 2, 2>(grid, a, sp, st);
        }
    }
    if (ms == 8) return launch_wide_ms<HZ, BITS, 8, 1>(grid, a, sp, st);
    if (ms == 4) return launch_wide_ms<HZ, BITS, 4, 1>(grid, a, sp, st);
    return launch_wide_ms<HZ, BITS, 2, 1>(grid, a, sp, st);
}

// Time of the plain fp16 4-bit launch: a block round costs s(rows) us per k-step, growing with
// the block count, one round per 256 blocks.  s = 0.62 / 0.92 / 1.57 us for 64- / 128- /
// 256-row tiles, fitted to MI355X measurements on the 7B-like prefill shapes for M = 48 .. 1024
// (within about 10 %).
double prefill_f16_estimate_us(const LinearArgs& a) {
    const bool offsets32 = (long long)a.M * a.K * 2 < (1LL << 31) && (long long)a.N * (a.K / 2) < (1LL << 31) &&
                           (long long)a.N * a.G * 2 < (1LL << 31);
    if (a.dtype != DT_F16 || a.K % (2 * W_BK) != 0 || !offsets32) return -1.0;
    const int ms = wide_ms(a.M, a.N);
    const long long blocks = wide_blocks(a.M, a.N, ms);
    const double s = ms == 2 ? 0.62 : (ms == 4 ? 0.92 : 1.57);
    const long long rounds = (blocks + 255) / 256;
    return s * (1.0 + (double)std::min(blocks, 256LL) / 1000.0) * (a.K / (double)W_BK) * (double)rounds;
}

bool prefill_supports(const LinearArgs& a) {
    if (a.dtype == DT_F16) return a.K % F_BK == 0 && a.g % F_BK == 0;   // any supported g
    return a.K % BK == 0 && a.g % BK == 0;
}

hipError_t launch_prefill(const LinearArgs& a, hipStream_t st) {
    const int hz = a.zeros ? 1 : 0;
    // the wide kernel addresses X, the packed weights and the group metadata with 32-bit
    // buffer offsets; larger operands take the 64-bit addressed kernel
    const bool offsets32 = (long long)a.M * a.K * 2 < (1LL << 31) && (long long)a.N * (a.K / 2) < (1LL << 31) &&
                           (long long)a.N * a.G * 2 < (1LL << 31);
    if (a.dtype == DT_F16 && a.K % (2 * W_BK) == 0 && offsets32)
        return hz ? launch_wide<true, 4>(a, st) : launch_wide<false, 4>(a, st);
    if (a.dtype == DT_F16) {
        const int tiles = ((a.M + F_BM - 1) / F_BM) * ((a.N + F_BN - 1) / F_BN);
        hipLaunchKernelGGL(prefill_f16_kernel, dim3(tiles), dim3(256), 0, st,
                           static_cast<const uint16_t*>(a.X), a.qw, a.scales, a.zeros, hz,
                           static_cast<uint16_t*>(a.Y), a.M, a.N, a.K, a.G, a.gshift);
        return hipGetLastError();
    }
    const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    const int spg = a.g / BK;
    hipLaunchKernelGGL(prefill_kernel<DT_BF16>, dim3(tiles), dim3(256), 0, st,
                       static_cast<const uint16_t*>(a.X), a.qw, a.scales, a.zeros, hz,
                       static_cast<uint16_t*>(a.Y), a.M, a.N, a.K, a.G, spg);
    return hipGetLastError();
}

// W8A16: the 128 x 128 tiled kernel with 8-bit codes, either dtype.
bool prefill8_supports(const LinearArgs& a) { return a.K % BK == 0 && a.g % BK == 0; }

hipError_t launch_prefill8(const LinearArgs& a, hipStream_t st) {
    if (!prefill8_supports(a)) return hipErrorInvalidValue;
    const int hz = a.zeros ? 1 : 0;
    // fp16: the wide kernel while its 32-bit buffer offsets cover the operands
    const bool offsets32 = (long long)a.M * a.K * 2 < (1LL << 31) && (long long)a.N * a.K < (1LL << 31) &&
                           (long long)a.N * a.G * 2 < (1LL << 31);
    if (a.dtype == DT_F16 && a.K % (2 * W_BK) == 0 && offsets32)
        return hz ? launch_wide<true, 8>(a, st) : launch_wide<false, 8>(a, st);
    const long long tiles = (long long)((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int spg = a.g / BK;
    if (a.dtype == DT_F16)
        hipLaunchKernelGGL((prefill_kernel<DT_F16, 8>), dim3((unsigned)tiles), dim3(256), 0, st,
                           static_cast<const uint16_t*>(a.X), a.qw, a.scales, a.zeros, hz,
                           static_cast<uint16_t*>(a.Y), a.M, a.N, a.K, a.G, spg);
    else
        hipLaunchKernelGGL((prefill_kernel<DT_BF16, 8>), dim3((unsigned)tiles), dim3(256), 0, st,
                           static_cast<const uint16_t*>(a.X), a.qw, a.scales, a.zeros, hz,
                           static_cast<uint16_t*>(a.Y), a.M, a.N, a.K, a.G, spg);
    return hipGetLastError();
}

}  // namespace w4a16
