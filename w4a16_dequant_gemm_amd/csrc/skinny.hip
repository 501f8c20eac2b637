// Small-batch W4A16 kernel on CDNA4 matrix cores (MFMA 16x16x32), 1 <= M <= 512.
//
// Decode batches are still bound by the weight stream (page "推理优化中“用精度换性能“的核心
// 技术：量化", section 一), but a VALU dot product costs one instruction per two weights
// per activation row, so beyond a couple of rows the arithmetic would outrun the
// stream.  Here the matrix cores do the multiply-adds for up to 16 activation rows per
// instruction and the VALU only unpacks codes (dequantization in registers, page
// "大模型推理中 Weight-only、W8A8 和 FP8 量化有什么区别？如何选型？", section 二).
//
// Work split.  A block of W waves owns NB row-blocks of 16 output rows, up to 32 activation
// rows (a second grid dimension runs over 32-row chunks of M) and all of K; wave w takes the
// k-blocks (128 columns each) w*KS .. w*KS + KS - 1 and streams them with two k-blocks in
// flight.  Partial 16x16 tiles are summed across the waves in LDS: the K split needs no
// buffer outside the block and no atomics, so results do not depend on scheduling.
//
// MFMA operands (lane l: n = l % 16, q = l / 16).
//   B (weights, 32 k x 16 n): lane (n, q) loads 16 bytes = 32 columns 32q .. 32q+31 of
//     the k-block from weight row n; MFMA j takes word j, columns 32q + 8j .. +7.  The
//     four MFMAs of a k-block stay inside its 128 columns, so any group size that is a
//     multiple of 128 (or the whole row) never splits an MFMA.
//   A (activations, 16 m x 32 k): lane (m, q) loads the same 8 columns of activation row
//     m; rows m >= M load through an out-of-range buffer offset, which returns zeros.
//   fp16: codes come out in natural column order as fp16 subnormals u * 2^-24 (byte
//     permutes with the constant-zero selector), so raw activations are the A operand.
//   bf16: codes are 128 + u in "byte order" (x0,x2)(x4,x6)(x1,x3)(x5,x7); the activation
//     fragment is permuted to match.
//   Zero point and bias leave through the activation group sums S, computed by the same
//   MFMA against a ones matrix: tile += s' * (acc - c * S) per k-block, fp16:
//   s' = s * 2^24, c = z (S in units of 2^-24); bf16: s' = s, c = 128 + z.
#include "common.h"
#include "launch.h"

namespace w4a16 {

namespace {

constexpr int kSkinnyWaves = 8;

template <int DT>
__device__ __forceinline__ f32x4 mfma16(const uint32_t a[4], const uint32_t b[4], f32x4 c) {
    if constexpr (DT == DT_F16) {
        f16x8 av, bv;
        __builtin_memcpy(&av, a, 16);
        __builtin_memcpy(&bv, b, 16);
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, c, 0, 0, 0);
    } else {
        bf16x8 av, bv;
        __builtin_memcpy(&av, a, 16);
        __builtin_memcpy(&bv, b, 16);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
    }
}

// fp16 codes in natural order: (u0,u1) (u2,u3) (u4,u5) (u6,u7) as subnormals.
__device__ __forceinline__ void unpack_natural_f16(uint32_t w, uint32_t out[4]) {
    const uint32_t t0 = w & 0x0F0F0F0Fu;           // u0 u2 u4 u6
    const uint32_t t1 = (w >> 4) & 0x0F0F0F0Fu;    // u1 u3 u5 u7
    // selector byte 0x0C yields a constant 0x00 byte
    out[0] = perm(t1, t0, 0x0C040C00u);
    out[1] = perm(t1, t0, 0x0C050C01u);
    out[2] = perm(t1, t0, 0x0C060C02u);
    out[3] = perm(t1, t0, 0x0C070C03u);
}

template <int NB, int MT>
struct KBlock {
    u32x4 a[MT][4];          // activation fragments, MFMA j
    u32x4 w[NB];             // 16 bytes of weights per row-block
    uint16_t s[NB], z[NB];
};

struct SkinnySrc {
    __amdgpu_buffer_rsrc_t x, w, s, z, none;
};

// SZL: the scales and zeros come from the block's LDS copy (row nb * 16 + n16 at stride gp)
// instead of two 2-byte loads per row-block and k-block.
template <int NB, int MT, bool SZL>
__device__ __forceinline__ void load_kblock(KBlock<NB, MT>& kb, const SkinnySrc& src, int k_block,
                                            bool live, const int va[MT], const int vw[NB],
                                            const int vs[NB], int gshift, const uint32_t* szl, int gp,
                                            int n16) {
    const __amdgpu_buffer_rsrc_t rx = live ? src.x : src.none;   // wave-uniform selects
    const __amdgpu_buffer_rsrc_t rw = live ? src.w : src.none;
    const __amdgpu_buffer_rsrc_t rs = live ? src.s : src.none;
    const __amdgpu_buffer_rsrc_t rz = live ? src.z : src.none;
    const int ox = k_block * 256;                          // 128 columns x 2 bytes
    const int ow = k_block * 64;                           // 128 columns x 4 bits
    const int og = ((k_block << 7) >> gshift) * 2;         // group of the k-block
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        kb.w[nb] = __builtin_amdgcn_raw_buffer_load_b128(rw, vw[nb], ow, 2 /* nt */);
        if constexpr (SZL) {
            const uint32_t v = szl[(nb * 16 + n16) * gp + ((k_block << 7) >> gshift)];
            kb.s[nb] = (uint16_t)v;
            kb.z[nb] = (uint16_t)(v >> 16);
        } else {
            kb.s[nb] = __builtin_amdgcn_raw_buffer_load_b16(rs, vs[nb], og, 0);
            kb.z[nb] = __builtin_amdgcn_raw_buffer_load_b16(rz, vs[nb], og, 0);
        }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            kb.a[mt][j] = __builtin_amdgcn_raw_buffer_load_b128(rx, va[mt] + 16 * j, ox, 0);
}

template <int DT, int NB, int MT>
__device__ __forceinline__ void compute_kblock(const KBlock<NB, MT>& kb, int has_zeros,
                                               f32x4 tile[NB][MT]) {
    const uint32_t one = DT == DT_F16 ? 0x00010001u : 0x3F803F80u;   // 2^-24 / 1.0 pairs
    const uint32_t ones[4] = {one, one, one, one};
    uint32_t a[MT][4][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4 v = kb.a[mt][j];
            if constexpr (DT == DT_F16) {
                a[mt][j][0] = v.x; a[mt][j][1] = v.y; a[mt][j][2] = v.z; a[mt][j][3] = v.w;
            } else {
                permute_x8_byte(v.x, v.y, v.z, v.w, a[mt][j]);
            }
        }
    // activation sums of the k-block, in the accumulator layout
    f32x4 S[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = mfma16<DT>(a[mt][j], ones, acc);
        S[mt] = acc;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        uint32_t b[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (DT == DT_F16)
                unpack_natural_f16(kb.w[nb][j], b[j]);
            else
                unpack_byte<0x43>(kb.w[nb][j], b[j]);
        }
        const float s = h2f(kb.s[nb]);
        const float z = has_zeros ? h2f(kb.z[nb]) : 8.0f;
        const float sp = DT == DT_F16 ? s * 16777216.0f : s;
        const float c = DT == DT_F16 ? z : 128.0f + z;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int j = 0; j < 4; ++j) acc = mfma16<DT>(a[mt][j], b[j], acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) tile[nb][mt][r] = fmaf(sp, fmaf(-c, S[mt][r], acc[r]), tile[nb][mt][r]);
        }
    }
}

template <int DT, int NB, int MT, int W, bool SZL>
__global__ __launch_bounds__(64 * W) void skinny_kernel(
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int has_zeros,
    uint16_t* __restrict__ Y, int M, int N, int K, int G, int gshift, int KS, int gp) {
    // the waves' partial tiles at the end; during the k-loop (SZL) the block's scales and zeros,
    // 16 NB rows x gp dwords (gp <= 16 W MT fits: the buffer holds W MT KB per row-block)
    __shared__ f32x4 red[W][NB][MT][64];
    uint32_t* szl = reinterpret_cast<uint32_t*>(&red[0][0][0][0]);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15;
    const int q = lane >> 4;
    const int KB = K >> 7;
    const int KW = K >> 3;
    const int row0 = blockIdx.x * (16 * NB);
    const int m0 = blockIdx.y * (16 * MT);              // this block's activation rows

    SkinnySrc src;
    src.x = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(X), 0, M * K * 2, 0x00020000);
    src.w = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(qw), 0, 0x7FFFFFFF, 0x00020000);
    src.s = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(scales), 0, 0x7FFFFFFF, 0x00020000);
    // NULL zeros: read the scales (valid memory); the value is replaced by 8
    src.z = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(has_zeros ? zeros : scales), 0,
                                              0x7FFFFFFF, 0x00020000);
    src.none = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(qw), 0, 0, 0x00020000);

    // Per-lane offsets that do not change along K.  Activation rows m >= M point past
    // the end of X (buffer range check: they read zeros); weight rows past N are clamped
    // (their results are not stored).
    int va[MT], vw[NB], vs[NB];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = m0 + mt * 16 + n16;
        va[mt] = m < M ? (m * K + 32 * q) * 2 : 0x7FFFFFF0;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int n = min(row0 + nb * 16 + n16, N - 1);
        vw[nb] = n * KW * 4 + 16 * q;
        vs[nb] = n * G * 2;
    }

    f32x4 tile[NB][MT];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) tile[nb][mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    if constexpr (SZL) {
        stage_sz_rows<4 * W / NB, 2 * W * MT>(szl, gp, tid, 16 * NB, row0, N, G, 0, G, has_zeros != 0, src.s, src.z,
                                              src.none);
        __syncthreads();
    }
    const int kb0 = wave * KS;
    const int kb1 = min(KB, kb0 + KS);
    const int nk = kb1 > kb0 ? kb1 - kb0 : 0;
    KBlock<NB, MT> buf0, buf1;
    load_kblock<NB, MT, SZL>(buf0, src, min(kb0, KB - 1), nk > 0, va, vw, vs, gshift, szl, gp, n16);
    load_kblock<NB, MT, SZL>(buf1, src, min(kb0 + 1, KB - 1), nk > 1, va, vw, vs, gshift, szl, gp, n16);
    // Unconditional prefetch and compute: a k-block past the end loads zeros through
    // `none` and adds nothing (zero activations, zero sums).
    for (int i = 0; i < nk; i += 2) {
        compute_kblock<DT, NB, MT>(buf0, has_zeros, tile);
        load_kblock<NB, MT, SZL>(buf0, src, min(kb0 + i + 2, KB - 1), i + 2 < nk, va, vw, vs, gshift, szl, gp, n16);
        compute_kblock<DT, NB, MT>(buf1, has_zeros, tile);
        load_kblock<NB, MT, SZL>(buf1, src, min(kb0 + i + 3, KB - 1), i + 3 < nk, va, vw, vs, gshift, szl, gp, n16);
    }
    if constexpr (SZL) __syncthreads();                  // every wave done with the staged words

    // Sum the waves' partial tiles; lane (n, q) of the tile holds rows m = 4q .. 4q+3.
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) red[wave][nb][mt][lane] = tile[nb][mt];
    __syncthreads();
    for (int e = tid; e < NB * MT * 64; e += 64 * W) {
        const int nb = e / (MT * 64);
        const int mt = (e / 64) % MT;
        const int l = e % 64;
        f32x4 v = red[0][nb][mt][l];
        for (int w = 1; w < W; ++w) {
            const f32x4 u = red[w][nb][mt][l];
            v[0] += u[0]; v[1] += u[1]; v[2] += u[2]; v[3] += u[3];
        }
        const int n = row0 + nb * 16 + (l & 15);
        if (n < N) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + mt * 16 + 4 * (l >> 4) + r;
                if (m < M) Y[(size_t)m * N + n] = f2out<DT>(v[r]);
            }
        }
    }
}

struct SkinnyCfg {
    int nb = 0, mt = 0, ks = 0, blocks = 0, mblocks = 1;
};

#ifndef W4A16_SKINNY_MAX_M
#define W4A16_SKINNY_MAX_M 512
#endif
constexpr int kSkinnyMaxM = W4A16_SKINNY_MAX_M;

SkinnyCfg pick_skinny(const LinearArgs& a) {
    SkinnyCfg c;
    c.mt = a.M > 32 ? 2 : (a.M + 15) / 16;
    // share activation fragments across two row-blocks when they are many, four past 32
    // activation rows (the grid then also runs over 32-row chunks of M, and each chunk's
    // activations are re-read once per 64 weight rows; the LDS reduction buffer,
    // W x NB x MT x 1 KB, stays within 64 KB)
    c.nb = a.M > 32 ? (a.dtype == DT_F16 ? 4 : 2) : (a.M > 8 ? 2 : 1);   // bf16 x4 would spill
    const int KB = a.K / 128;
    c.ks = (KB + kSkinnyWaves - 1) / kSkinnyWaves;
    c.blocks = (a.N + 16 * c.nb - 1) / (16 * c.nb);
    c.mblocks = (a.M + 16 * c.mt - 1) / (16 * c.mt);
    return c;
}

template <int DT, int NB, int MT>
hipError_t run(const LinearArgs& a, const SkinnyCfg& c, hipStream_t st) {
    // scales and zeros staged in LDS when the row's groups fit the reduction buffer (gp = G | 1
    // <= 16 W MT words per row: G < 128 MT); measured (fp16, g = 128): M = 256, 11008 -> 4096:
    // 109.5 -> 92.4 us; M = 128, 4096 -> 4096: 24.2 -> 18.1 us; M = 32, 4096 -> 11008: 31.6 ->
    // 25.7 us (the address unit was 75 % busy)
    const bool szl = (a.G | 1) <= 16 * kSkinnyWaves * MT;
    if (szl)
        hipLaunchKernelGGL((skinny_kernel<DT, NB, MT, kSkinnyWaves, true>), dim3(c.blocks, c.mblocks),
                           dim3(64 * kSkinnyWaves), 0, st, static_cast<const uint16_t*>(a.X), a.qw,
                           a.scales, a.zeros, a.zeros ? 1 : 0, static_cast<uint16_t*>(a.Y), a.M, a.N,
                           a.K, a.G, a.gshift, c.ks, a.G | 1);
    else
        hipLaunchKernelGGL((skinny_kernel<DT, NB, MT, kSkinnyWaves, false>), dim3(c.blocks, c.mblocks),
                           dim3(64 * kSkinnyWaves), 0, st, static_cast<const uint16_t*>(a.X), a.qw,
                           a.scales, a.zeros, a.zeros ? 1 : 0, static_cast<uint16_t*>(a.Y), a.M, a.N,
                           a.K, a.G, a.gshift, c.ks, 0);
    return hipGetLastError();
}

template <int DT>
hipError_t run_dt(const LinearArgs& a, const SkinnyCfg& c, hipStream_t st) {
    if (c.nb == 1 && c.mt == 1) return run<DT, 1, 1>(a, c, st);
    if (c.nb == 2 && c.mt == 1) return run<DT, 2, 1>(a, c, st);
    if (c.nb == 2 && c.mt == 2) return run<DT, 2, 2>(a, c, st);
    if constexpr (DT == DT_F16)
        if (c.nb == 4 && c.mt == 2) return run<DT, 4, 2>(a, c, st);
    return hipErrorInvalidValue;
}

}  // namespace

bool skinny_supports(const LinearArgs& a) {
    if (a.M < 1 || a.M > kSkinnyMaxM) return false;
    if (a.K % 128 != 0) return false;
    if (a.g % 128 != 0) return false;             // g == K qualifies when K % 128 == 0
    // 32-bit buffer offsets
    if ((long long)a.N * (a.K / 2) >= (1LL << 31) || (long long)a.M * a.K * 2 >= (1LL << 31))
        return false;
    return true;
}

hipError_t launch_skinny(const LinearArgs& a, hipStream_t st) {
    if (decode_supports(a)) return launch_decode(a, st);     // 1 <= M <= 4
    const SkinnyCfg c = pick_skinny(a);
    return a.dtype == DT_F16 ? run_dt<DT_F16>(a, c, st) : run_dt<DT_BF16>(a, c, st);
}

}  // namespace w4a16
