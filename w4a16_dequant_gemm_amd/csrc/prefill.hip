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
// fp16 kernel: dequantize once per block into LDS.
//
// Block tile 256 (M) x 128 (N), k-step 32, 256 threads = 4 waves in a 2 x 2 grid, wave
// tile 128 x 64 = 4 x 2 MFMA 32x32x16 tiles.  Per k-step every thread
//   - loads 64 bytes of one activation row (its 32 columns) and stores them to LDS
//     unchanged (natural column order),
//   - loads 8 bytes = 16 codes of one weight row and writes the dequantized fp16 weights
//     s * (u - z) to LDS: the code pair (u, u') is built as the fp16 bits of
//     1536 + (u - z) by one packed 16-bit integer add (exact while |u - z| < 512), then
//     1536 is subtracted (exact) and the pair is multiplied by s (one rounding),
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
    // dequantization constants of the current group: (0x6600 - z) pair and s pair
    uint32_t zbias = 0, spair = 0;
    int cur_group = -1;
    auto store_step = [&](int buf, int step) {
        const int grp = group_of(step * F_BK, gshift);
        if (grp != cur_group) {
            cur_group = grp;
            const uint16_t sb = scales[(size_t)wrow * G + grp];
            const float z = has_zeros ? h2f(zsrc[(size_t)wrow * G + grp]) : 8.0f;
            const uint32_t zb = (uint32_t)(0x6600 - (int)z) & 0xFFFFu;
            zbias = zb | (zb << 16);
            spair = (uint32_t)sb | ((uint32_t)sb << 16);
        }
        uint16_t* arow = &As[buf][tid * F_LDA];
#pragma unroll
        for (int b = 0; b < 4; ++b) *reinterpret_cast<u32x4*>(arow + 8 * b) = xa[b];
        const f16x2 bias = {(_Float16)1536.0f, (_Float16)1536.0f};
        const f16x2 sv = __builtin_bit_cast(f16x2, spair);
        uint32_t d[8];
#pragma unroll
        for (int wi = 0; wi < 2; ++wi) {
            const uint32_t w = wq[wi];
            const uint32_t t0 = w & 0x0F0F0F0Fu;          // u0 u2 u4 u6 (as bytes)
            const uint32_t t1 = (w >> 4) & 0x0F0F0F0Fu;   // u1 u3 u5 u7
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                // (u_{2p}, u_{2p+1}) as 16-bit integers, then the fp16 bits of 1536 + u - z
                const uint32_t uu = perm(t1, t0, 0x0C040C00u + 0x00010001u * p);
                const uint32_t biased = __builtin_bit_cast(uint32_t,
                    __builtin_bit_cast(u16x2, uu) + __builtin_bit_cast(u16x2, zbias));
                const f16x2 code = __builtin_bit_cast(f16x2, biased) - bias;    // exact
                d[4 * wi + p] = __builtin_bit_cast(uint32_t, code * sv);        // one rounding
            }
        }
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
//     step ahead, and turns word j into the fp16 B fragment of MFMA j with the 1536-bias
//     construction (exact 1536 + u - z, exact subtraction, one rounding in the multiply
//     by s).  MFMA j covers columns 8 j .. 8 j + 7 and 32 + 8 j .. + 7; the activation
//     fragment of lane (m, h) reads the same columns.  The next step's dequantization is
//     interleaved with this step's MFMAs.
//   Block order: consecutive block indices run on different XCDs; blocks are renumbered
//     so that each XCD works through consecutive tiles (a few 256-row activation panels,
//     held in that XCD's L2).
constexpr int W_BM = 256, W_BN = 256, W_BK = 64;     // K % 128 == 0: steps in pairs

// BITS = 8 (W8A16): lane (n, h) loads the 32 bytes of columns 32h .. 32h + 31 (two 16-byte
// loads) and MFMA j takes words 2j and 2j + 1 (one byte permute per pair instead of the nibble
// masks; the 1536-bias construction is exact for |u - z| < 512, the implicit symmetric zero
// point is 128).
// Split K (part != NULL): block (x, y) runs k-steps [y * spl, (y + 1) * spl) of its tile and
// stores the fp32 partial tile to part[y][M][N]; splitk_reduce_kernel sums the partials in
// split order.  Without a split, spl = K / 64, grid y = 1 and the tile goes to Y.
template <bool HZ, int BITS = 4, bool SPLIT = false>
__global__ __launch_bounds__(256, 1) void prefill_f16_wide_kernel(
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros,
    uint16_t* __restrict__ Y, int M, int N, int K, int G, int gshift,
    float* __restrict__ part = nullptr, int spl = 0) {
    __shared__ __attribute__((aligned(16))) u32x4 As[2][W_BM * 8];     // 2 x 32 KB

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int h = lane >> 5;
    int mt, nt;
    if (!xcd_tile(blockIdx.x, (M + W_BM - 1) / W_BM, (N + W_BN - 1) / W_BN, mt, nt)) return;
    const int m0 = mt * W_BM;
    const int n0 = nt * W_BN;
    const int nsteps = K / W_BK;
    const int sb = SPLIT ? blockIdx.y * spl : 0;          // this block's k-steps [sb, se), even count
    const int se = SPLIT ? min(nsteps, sb + spl) : nsteps;
    if constexpr (SPLIT) {
        if (sb >= se) return;                             // never planned (every split has steps)
    }

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

    // activation staging: instruction j of wave w fills slots (8 w + j) * 64 + lane, i.e.
    // row r = (8 w + j) * 8 + lane / 8, slot lane % 8, which holds column piece
    // (lane % 8) ^ ((r / 2) % 8)
    int xoff[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int r = (8 * wave + j) * 8 + (lane >> 3);
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
    auto load_a = [&](int buf, int step) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rx, (__attribute__((address_space(3))) void*)&As[buf][(8 * wave + j) * 64], 16,
                xoff[j], step * W_BK * 2, 0, 0);
    };
    constexpr int WL = BITS == 4 ? 1 : 2;        // 16-byte weight loads per row and step
    struct WStage {
        u32x4 w[2][WL];
        uint16_t s[2], z[2];
    };
    auto load_w = [&](WStage& st, int step) {
        const int grp2 = group_of(step * W_BK + 32 * h, gshift) * 2;
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) {
#pragma unroll
            for (int i = 0; i < WL; ++i)
                st.w[ns][i] = __builtin_amdgcn_raw_buffer_load_b128(rw, woff[ns] + 16 * i, step * (W_BK / 8 * BITS), 0);
            st.s[ns] = __builtin_amdgcn_raw_buffer_load_b16(rs, szoff[ns] + grp2, 0, 0);
            st.z[ns] = __builtin_amdgcn_raw_buffer_load_b16(rz, szoff[ns] + grp2, 0, 0);
        }
    };
    // word j of both rows of a stage -> the fp16 B fragments of MFMA j: b[ns][j][4]
    auto dequant_word = [&](const WStage& st, int j, uint32_t b[2][4][4]) {
        const f16x2 bias = {(_Float16)1536.0f, (_Float16)1536.0f};
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) {
            const float z = HZ ? h2f(st.z[ns]) : (BITS == 4 ? 8.0f : 128.0f);
            const uint32_t zb = (uint32_t)(0x6600 - (int)z) & 0xFFFFu;
            const u16x2 zbias = __builtin_bit_cast(u16x2, zb | (zb << 16));
            const f16x2 sv = __builtin_bit_cast(f16x2, (uint32_t)st.s[ns] | ((uint32_t)st.s[ns] << 16));
            uint32_t t0, t1;
            if constexpr (BITS == 4) {
                const uint32_t w = st.w[ns][0][j];
                t0 = w & 0x0F0F0F0Fu;                     // u0 u2 u4 u6 (as bytes)
                t1 = (w >> 4) & 0x0F0F0F0Fu;              // u1 u3 u5 u7
            } else {
                t0 = st.w[ns][j >> 1][2 * (j & 1)];       // bytes u0 u1 u2 u3
                t1 = st.w[ns][j >> 1][2 * (j & 1) + 1];   // bytes u4 u5 u6 u7
            }
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                uint32_t uu;                               // (u_2p, u_2p+1) as 16-bit integers
                if constexpr (BITS == 4)
                    uu = perm(t1, t0, 0x0C040C00u + 0x00010001u * p);
                else
                    uu = p < 2 ? perm(0u, t0, 0x0C010C00u + 0x00020002u * p)
                               : perm(0u, t1, 0x0C010C00u + 0x00020002u * (p - 2));
                const u16x2 biased = __builtin_bit_cast(u16x2, uu) + zbias;     // 1536 + u - z
                const f16x2 code = __builtin_bit_cast(f16x2, biased) - bias;    // exact
                b[ns][j][p] = __builtin_bit_cast(uint32_t, code * sv);          // one rounding
            }
        }
    };

    f32x16 acc[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i)
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
    auto compute = [&](int buf, const uint32_t bc[2][4][4], const WStage& nx, uint32_t bn[2][4][4]) {
        const u32x4* A = As[buf];
        u32x4 fa[8], fb[8];        // activation fragments one MFMA group ahead
#pragma unroll
        for (int ms = 0; ms < 8; ++ms) fa[ms] = A[ms * 256 + fslot[0]];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x4* cur = (j & 1) ? fb : fa;
            u32x4* nxt = (j & 1) ? fa : fb;
            if (j < 3) {
#pragma unroll
                for (int ms = 0; ms < 8; ++ms) nxt[ms] = A[ms * 256 + fslot[j + 1]];
            }
#pragma unroll
            for (int ms = 0; ms < 8; ++ms) {
                const uint32_t af[4] = {cur[ms].x, cur[ms].y, cur[ms].z, cur[ms].w};
#pragma unroll
                for (int ns = 0; ns < 2; ++ns) acc[ms][ns] = Mfma<DT_F16>::run(af, bc[ns][j], acc[ms][ns]);
            }
            dequant_word(nx, j, bn);
            // interleave: one fragment read and a few dequant instructions per MFMA pair
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (j < 3) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);              // VALU
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // MFMA
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Pipeline: activations one step ahead (global -> LDS), packed weights one step ahead
    // and dequantized weights one step ahead (registers).  The LDS-destination loads are
    // complete when vmcnt drains; each step ends with that wait and a barrier.  Loads past
    // the last step re-read it (harmless, unused).
    WStage p0, p1;
    uint32_t b0[2][4][4], b1[2][4][4];
    load_a(0, sb);
    load_w(p0, sb);
    load_w(p1, min(sb + 1, se - 1));
#pragma unroll
    for (int j = 0; j < 4; ++j) dequant_word(p0, j, b0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int step = sb; step < se; step += 2) {
        load_a(1, min(step + 1, se - 1));
        load_w(p0, min(step + 2, se - 1));
        compute(0, b0, p1, b1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        load_a(0, min(step + 2, se - 1));
        load_w(p1, min(step + 3, se - 1));
        compute(1, b1, p0, b0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

#pragma unroll
    for (int ms = 0; ms < 8; ++ms) {
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
    if (a.zeros)
        hipLaunchKernelGGL((prefill_f16_wide_kernel<true, 4, true>), grid, dim3(256), 0, st,
                           static_cast<const uint16_t*>(a.X), a.qw, a.scales, a.zeros, static_cast<uint16_t*>(a.Y),
                           a.M, a.N, a.K, a.G, a.gshift, work, spl);
    else
        hipLaunchKernelGGL((prefill_f16_wide_kernel<false, 4, true>), grid, dim3(256), 0, st,
                           static_cast<const uint16_t*>(a.X), a.qw, a.scales, a.zeros, static_cast<uint16_t*>(a.Y),
                           a.M, a.N, a.K, a.G, a.gshift, work, spl);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long MN = (long long)a.M * a.N;
    const long long blocks = (MN + 255) / 256;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, st,
                       work, S, MN, static_cast<uint16_t*>(a.Y));
    return hipGetLastError();
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
    if (a.dtype == DT_F16 && a.K % (2 * W_BK) == 0 && offsets32) {
        const int tiles = ((a.M + W_BM - 1) / W_BM) * ((a.N + W_BN - 1) / W_BN);
        const int grid = 8 * ((tiles + 7) / 8);
        if (hz)
            hipLaunchKernelGGL(prefill_f16_wide_kernel<true>, dim3(grid), dim3(256), 0, st,
                               static_cast<const uint16_t*>(a.X), a.qw, a.scales, a.zeros,
                               static_cast<uint16_t*>(a.Y), a.M, a.N, a.K, a.G, a.gshift);
        else
            hipLaunchKernelGGL(prefill_f16_wide_kernel<false>, dim3(grid), dim3(256), 0, st,
                               static_cast<const uint16_t*>(a.X), a.qw, a.scales, a.zeros,
                               static_cast<uint16_t*>(a.Y), a.M, a.N, a.K, a.G, a.gshift);
        return hipGetLastError();
    }
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
    // fp16: the 256 x 256 kernel while its 32-bit buffer offsets cover the operands
    const bool offsets32 = (long long)a.M * a.K * 2 < (1LL << 31) && (long long)a.N * a.K < (1LL << 31) &&
                           (long long)a.N * a.G * 2 < (1LL << 31);
    if (a.dtype == DT_F16 && a.K % (2 * W_BK) == 0 && offsets32) {
        const int tiles = ((a.M + W_BM - 1) / W_BM) * ((a.N + W_BN - 1) / W_BN);
        const int grid = 8 * ((tiles + 7) / 8);
        if (hz)
            hipLaunchKernelGGL((prefill_f16_wide_kernel<true, 8>), dim3(grid), dim3(256), 0, st,
                               static_cast<const uint16_t*>(a.X), a.qw, a.scales, a.zeros,
                               static_cast<uint16_t*>(a.Y), a.M, a.N, a.K, a.G, a.gshift);
        else
            hipLaunchKernelGGL((prefill_f16_wide_kernel<false, 8>), dim3(grid), dim3(256), 0, st,
                               static_cast<const uint16_t*>(a.X), a.qw, a.scales, a.zeros,
                               static_cast<uint16_t*>(a.Y), a.M, a.N, a.K, a.G, a.gshift);
        return hipGetLastError();
    }
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
