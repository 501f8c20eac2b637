// Decode-regime W4A16 kernel: weight-streaming GEMV for small M (v_dot2 on the VALU).
//
// At decode the layer reads every weight once per token and does two flops per weight
// per activation row, so it is bound by the weight stream from HBM, not by arithmetic
// (page "推理优化中“用精度换性能“的核心技术：量化", section 一; page
// "Quantization & Acceleration: 解释 W8A8 与 W4A16 的差异与取舍", decode vs prefill).  The
// kernel (i) reads each packed weight row exactly once with coalesced 128-bit loads, all
// issued before any arithmetic so the whole per-block share of the stream is in flight
// at once, (ii) dequantizes in registers only (page
// "大模型推理中 Weight-only、W8A8 和 FP8 量化有什么区别？如何选型？", section 二) and
// (iii) keeps the activations in registers.
//
// Mapping.  A block of NT threads (a multiple of 64) owns RB consecutive output rows and
// the whole K range.  Thread t owns the 32-column chunks c = t + NT*i (i < CPL) of every
// row; a 16-byte chunk never straddles a group (g is a multiple of 32), so each chunk
// contributes s * (sum x*u - z * sum x) with one scale and one zero point.
//   fp16: codes are fp16 subnormals from two masks (unpack_mask_f16); the x1 and x16
//     pairs go to two v_dot2 accumulators; 2^24 is folded into the scale.
//   bf16: codes are 128 + u from byte permutes (unpack_byte<0x43>); the bias leaves with
//     the chunk's activation sum.
// Partial sums are reduced across the wave with DPP and across waves through LDS.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace w4a16 {

namespace {

// Conservative VGPR estimate of one configuration; it decides the launch bound.
constexpr int gemv_regs(int M, int CPL, int RB) {
    return 6 * RB * CPL + 16 * M * CPL + 3 * RB * M + 40;
}
constexpr int launch_limit(int M, int CPL, int RB) {
    return gemv_regs(M, CPL, RB) <= 128 ? 1024 : (gemv_regs(M, CPL, RB) <= 256 ? 512 : 0);
}

template <int DT, int M, int CPL, int RB>
__global__ __launch_bounds__(launch_limit(M, CPL, RB)) void gemv_kernel(
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int has_zeros,
    uint16_t* __restrict__ Y, int N, int K, int G, int gshift) {
    __shared__ float red[16][RB * M];
    const int tid = threadIdx.x;
    const int NT = blockDim.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nwaves = NT >> 6;
    const int C = K >> 5;
    const int KW = K >> 3;
    const int row0 = blockIdx.x * RB;
    // A NULL zero-point array reads the scales instead (always valid memory); the value
    // is replaced by 8 below.  Keeps every load unconditional.
    const uint16_t* zsrc = has_zeros ? zeros : scales;

    int cc[CPL], cg[CPL];
    bool cval[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = tid + NT * i;
        cval[i] = c < C;
        cc[i] = cval[i] ? c : 0;      // chunks past the row end re-read chunk 0 ...
        cg[i] = group_of(cc[i] << 5, gshift);
    }

    // 1. Activations first (vmcnt waits are in issue order and they are needed first),
    //    then the whole weight share of this block.  Rows past N are clamped to N-1 (their
    //    results are not stored).
    u32x4 xv[M][CPL][4];
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                xv[m][i][b] = reinterpret_cast<const u32x4*>(X + (size_t)m * K + ((size_t)cc[i] << 5))[b];
    u32x4 wv[RB][CPL];
    uint16_t sraw[RB][CPL], zraw[RB][CPL];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const int n = min(row0 + r, N - 1);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            wv[r][i] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(qw + (size_t)n * KW + ((size_t)cc[i] << 2)));
            sraw[r][i] = scales[(size_t)n * G + cg[i]];
            zraw[r][i] = zsrc[(size_t)n * G + cg[i]];
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2. Activations to pair order; chunk sums.  ... and get zero activations, so they
    //    contribute nothing whatever weights they meet.
    uint32_t xr[M][CPL][16];
    float xs[M][CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float sum = 0.0f;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const u32x4 v = xv[m][i][b];
                uint32_t o[4];
                if constexpr (DT == DT_F16)
                    permute_x8(v.x, v.y, v.z, v.w, o);
                else
                    permute_x8_byte(v.x, v.y, v.z, v.w, o);
#pragma unroll
                for (int q = 0; q < 4; ++q) xr[m][i][4 * b + q] = cval[i] ? o[q] : 0u;
                sum += (pair_sum<DT>(v.x) + pair_sum<DT>(v.y)) + (pair_sum<DT>(v.z) + pair_sum<DT>(v.w));
            }
            // fp16 works in units of 2^-24 (the subnormal code scale)
            xs[m][i] = cval[i] ? (DT == DT_F16 ? sum * 5.9604644775390625e-8f : sum) : 0.0f;
        }
    }

    // 3. Dot products.
    float acc[RB][M];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const float s = h2f(sraw[r][i]);
            const float z = has_zeros ? h2f(zraw[r][i]) : 8.0f;
            if constexpr (DT == DT_F16) {
                float pa[M], pb[M];
#pragma unroll
                for (int m = 0; m < M; ++m) pa[m] = pb[m] = 0.0f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    uint32_t cd[4];
                    unpack_mask_f16(wv[r][i][q], cd);
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        pa[m] = dot2<DT>(xr[m][i][4 * q + 0], cd[0], pa[m]);
                        pb[m] = dot2<DT>(xr[m][i][4 * q + 1], cd[1], pb[m]);
                        pa[m] = dot2<DT>(xr[m][i][4 * q + 2], cd[2], pa[m]);
                        pb[m] = dot2<DT>(xr[m][i][4 * q + 3], cd[3], pb[m]);
                    }
                }
                const float s24 = s * 16777216.0f;     // 2^24: exact
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    float t = fmaf(pb[m], 0.0625f, pa[m]);   // sum x*u * 2^-24
                    t = fmaf(-z, xs[m][i], t);
                    acc[r][m] = fmaf(s24, t, acc[r][m]);
                }
            } else {
                float p[M];
#pragma unroll
                for (int m = 0; m < M; ++m) p[m] = 0.0f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    uint32_t cd[4];
                    unpack_byte<0x43>(wv[r][i][q], cd);
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        p[m] = dot2<DT>(xr[m][i][4 * q + 0], cd[0], p[m]);
                        p[m] = dot2<DT>(xr[m][i][4 * q + 1], cd[1], p[m]);
                        p[m] = dot2<DT>(xr[m][i][4 * q + 2], cd[2], p[m]);
                        p[m] = dot2<DT>(xr[m][i][4 * q + 3], cd[3], p[m]);
                    }
                }
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const float t = fmaf(-(128.0f + z), xs[m][i], p[m]);
                    acc[r][m] = fmaf(s, t, acc[r][m]);
                }
            }
        }
    }

    // 4. Reduce over the wave (DPP) and over the waves (LDS); round once to the output.
    if (nwaves == 1) {
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const float v = wave_sum(acc[r][m]);
                if (lane == 0 && row0 + r < N) Y[(size_t)m * N + row0 + r] = f2out<DT>(v);
            }
        return;
    }
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const float v = wave_sum(acc[r][m]);
            if (lane == 0) red[wave][r * M + m] = v;
        }
    __syncthreads();
    if (tid < RB * M) {
        const int r = tid / M;
        const int m = tid % M;
        float v = 0.0f;
        for (int w = 0; w < nwaves; ++w) v += red[w][tid];
        if (row0 + r < N) Y[(size_t)m * N + row0 + r] = f2out<DT>(v);
    }
}

// ---------------------------------------------------------------------------------
// Streaming variant (used whenever the activations fit in LDS).  The grid is a fixed,
// balanced set of persistent blocks: block b owns a contiguous range of about N / grid
// rows.  The block stages the permuted activations and their 32-column chunk sums in
// LDS once; then wave w of the block walks the rows row_begin + w*RB + i*W*RB
// (batches of RB rows), lane l handling chunks l + 64 c of each row.  Weight loads of
// the next batch are issued before the current batch is computed (two register
// buffers), so the arithmetic of one batch overlaps the HBM stream of the next.  Each
// wave owns whole rows: one DPP reduction per row, no cross-wave traffic.
constexpr int kLdsBudget = 65536;

// Staged activations: per row, four planes (one per 16-byte piece of a 32-column chunk) of
// CPL * 64 chunk slots plus one pad slot, so that the four lanes staging one chunk write four
// different banks (planes exactly CPL * 1 KB apart put all four in the same banks); then one
// spare slot, then the chunk sums (M * CPL * 64 + 1 floats).
__host__ __device__ constexpr int x_plane(int CPL) { return CPL * 64 + 1; }
__host__ __device__ constexpr int x_slots(int M, int CPL) { return 4 * M * x_plane(CPL) + 1; }
__host__ __device__ constexpr int lds_bytes(int M, int CPL) { return x_slots(M, CPL) * 16 + (M * CPL * 64 + 1) * 4; }

template <int DT, int M, int CPL, int RB>
struct RowBatch {
    u32x4 w[RB][CPL];
};

// Buffer loads: the row offset is wave-uniform (an SGPR soffset) and the lane's chunk
// offset never changes between rows (voffset), so a load costs no address arithmetic.
// A batch past the wave's last one loads through `none` (num_records = 0): buffer loads
// out of range return zeros without touching memory, so every prefetch can be issued
// unconditionally.
struct StreamSrc {
    __amdgpu_buffer_rsrc_t w, s, z, none;
    int row_bytes_w;
};

// CLIP: rows at or past `row_lim` (another wave's) load zeros through `none`; otherwise
// rows are clamped to row_lim - 1 (rows past the block's end re-read valid memory and their
// results are not stored).
template <int DT, int M, int CPL, int RB, bool CLIP>
__device__ __forceinline__ void load_batch(RowBatch<DT, M, CPL, RB>& bt, const StreamSrc& src, int row,
                                           bool live, int row_lim, const int vw[CPL]) {
    const __amdgpu_buffer_rsrc_t rw = live ? src.w : src.none;   // wave-uniform select
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            if constexpr (CLIP) {
                const bool in = live && row + r < row_lim;              // wave-uniform
                bt.w[r][i] = __builtin_amdgcn_raw_buffer_load_b128(in ? src.w : src.none, vw[i],
                                                                   (in ? row + r : 0) * src.row_bytes_w, 2);
            } else {
                const int n = min(row + r, row_lim - 1);                // wave-uniform
                bt.w[r][i] = __builtin_amdgcn_raw_buffer_load_b128(rw, vw[i], n * src.row_bytes_w, 2 /* nt */);
            }
        }
    }
}

// szl: the block's group factors, one (s', c) float pair per (row, group), rows relative
// to the block (szrow = index of the batch's first row): a chunk adds s' * P + c * S to
// its row (P its dot product, S its activation sum); fp16: s' = s * 2^24, c = -z * s'
// (P and S in units of 2^-24); bf16: s' = s, c = -(128 + z) * s.  Both are exact in fp32.
template <int DT, int M, int CPL, int RB>
__device__ __forceinline__ void compute_batch(const RowBatch<DT, M, CPL, RB>& bt, const uint32_t* xp,
                                              const float* xsum, const float2* szl, int szrow, int G,
                                              int nrows, const int lgrp[CPL], int C, int gshift, int lane,
                                              float acc[RB][M]) {
    constexpr int CH = CPL * 64;
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        uint32_t xr[M][16];
        float xs[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            // piece-major layout [m][piece][chunk]: a wave reads 64 consecutive 16-byte slots
            const u32x4* src = reinterpret_cast<const u32x4*>(xp) + (size_t)m * 4 * x_plane(CPL) + c;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const u32x4 v = src[b * x_plane(CPL)];
                xr[m][4 * b + 0] = v.x;
                xr[m][4 * b + 1] = v.y;
                xr[m][4 * b + 2] = v.z;
                xr[m][4 * b + 3] = v.w;
            }
            xs[m] = xsum[m * CH + c];
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            // rows past the batch's last real row (zeros loaded, result not stored) read
            // that row's factors, so every LDS read stays inside the staged words
            // one row: recomputed, so that no register holds it across the loads (the grouped
            // kernel's allocation stays at 64 VGPRs); more rows: kept, as recomputing cost more
            const int grp = M == 1 ? group_of((c < C ? c : 0) << 5, gshift) : lgrp[i];
            const float2 f = szl[szrow + (r < nrows ? r : nrows - 1) * G + grp];
            if constexpr (DT == DT_F16) {
                float pa[M], pb[M];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    uint32_t cd[4];
                    unpack_mask_f16(bt.w[r][i][q], cd);
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        pa[m] = dot2<DT>(xr[m][4 * q + 0], cd[0], q == 0 ? 0.0f : pa[m]);
                        pb[m] = dot2<DT>(xr[m][4 * q + 1], cd[1], q == 0 ? 0.0f : pb[m]);
                        pa[m] = dot2<DT>(xr[m][4 * q + 2], cd[2], pa[m]);
                        pb[m] = dot2<DT>(xr[m][4 * q + 3], cd[3], pb[m]);
                    }
                }
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const float t = fmaf(pb[m], 0.0625f, pa[m]);     // sum x*u * 2^-24
                    acc[r][m] = fmaf(f.y, xs[m], fmaf(f.x, t, acc[r][m]));
                }
            } else {
                float p[M];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    uint32_t cd[4];
                    unpack_byte<0x43>(bt.w[r][i][q], cd);
#pragma unroll
                    for (int m = 0; m < M; ++m) {
                        p[m] = dot2<DT>(xr[m][4 * q + 0], cd[0], q == 0 ? 0.0f : p[m]);
                        p[m] = dot2<DT>(xr[m][4 * q + 1], cd[1], p[m]);
                        p[m] = dot2<DT>(xr[m][4 * q + 2], cd[2], p[m]);
                        p[m] = dot2<DT>(xr[m][4 * q + 3], cd[3], p[m]);
                    }
                }
#pragma unroll
                for (int m = 0; m < M; ++m) acc[r][m] = fmaf(f.y, xs[m], fmaf(f.x, p[m], acc[r][m]));
            }
        }
        __builtin_amdgcn_sched_barrier(0);   // one chunk of activations live at a time
    }
}

// Rows at or past row_end belong to the next block (or do not exist) and are not stored.
template <int DT, int M, int RB>
__device__ __forceinline__ void store_batch(const float acc[RB][M], int row, int row_end, int N,
                                            int lane, uint16_t* __restrict__ Y) {
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        if (row + r >= row_end) break;                 // wave-uniform
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const float v = wave_sum(acc[r][m]);
            if (lane == 0) Y[(size_t)m * N + row + r] = f2out<DT>(v);
        }
    }
}

// Byte offset of the (scale, zero point) words in the stream kernel's LDS.
__host__ __device__ constexpr int sz_lds_offset(int M, int CPL) { return (lds_bytes(M, CPL) + 15) & ~15; }
constexpr int kSzPiecesPerThread = 2;     // 16-byte pieces of scales (and of zeros) per thread

// The work of one block of the streaming kernel (block index `blk`), shared by the plain
// kernel and the grouped kernel (several independent layers in one launch).  JSZ: 16-byte
// pieces of scales (and of zeros) each thread stages; the launcher checks that the block's
// pieces fit.
template <int DT, int M, int CPL, int RB, int W, int NB, int JSZ>
__device__ __forceinline__ void stream_block(
    uint32_t* __restrict__ lds, const uint16_t* __restrict__ X, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int has_zeros,
    uint16_t* __restrict__ Y, int N, int K, int G, int gshift, int rows_per_block, int blk) {
    constexpr int CH = CPL * 64;                       // padded chunks per activation row
    constexpr int NT = 64 * W;
    constexpr int JOBS = M * CH * 4;                   // 8-column staging jobs
    constexpr int JPT = (JOBS + NT - 1) / NT;
    constexpr int PS = x_plane(CPL);                   // slots per piece plane (one pad slot)
    uint32_t* xp = lds;                  // [M][4 pieces][PS] x 16 B pairs, then one spare slot
    float* xsum = reinterpret_cast<float*>(lds + x_slots(M, CPL) * 4);   // [M*CH + 1]
    float2* szs = reinterpret_cast<float2*>(lds + sz_lds_offset(M, CPL) / 4);   // staged group factors
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int C = K >> 5;
    const int KW = K >> 3;
    const int row_begin = blk * rows_per_block;
    const int row_end = min(N, row_begin + rows_per_block);
    // NB == 0: one batch per wave holding all of its rows, an even split of the block's
    // rows (wave w: rows_w .. rows_{w+1} - 1); otherwise batches of RB rows strided by W * RB.
    constexpr bool ONE = NB == 0;
    constexpr int NBUF = ONE ? 1 : NB;
    const int nrows_blk = row_end - row_begin;
    const int first = ONE ? row_begin + (wave * nrows_blk) / W : row_begin + wave * RB;
    const int wave_end = ONE ? row_begin + ((wave + 1) * nrows_blk) / W : row_end;
    const int nbatch = ONE ? (first < wave_end ? 1 : 0)
                           : (first < row_end ? (row_end - first + W * RB - 1) / (W * RB) : 0);

    // The block's scales (and zeros) are one contiguous run of (row_end - row_begin) * G
    // halves; it is staged in 16-byte pieces from the 16-byte boundary at or below its
    // start.  Pieces that lie wholly inside the arrays are loaded with 16-byte loads; the
    // last (N * G) % 8 halves of the arrays, if any, with 2-byte loads.
    const int total = N * G;
    const int full_end = total & ~7;
    StreamSrc src;
    src.w = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(qw), 0, 0x7FFFFFFF, 0x00020000);
    // NULL zeros: read the scales (valid memory); the value is replaced by 8
    const uint16_t* zsrc = has_zeros ? zeros : scales;
    src.s = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(scales), 0, full_end * 2, 0x00020000);
    src.z = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(zsrc), 0, full_end * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t s_all =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(scales), 0, total * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t z_all =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(zsrc), 0, total * 2, 0x00020000);
    src.none = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(qw), 0, 0, 0x00020000);
    src.row_bytes_w = KW * 4;
    int vw[CPL], lgrp[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int c = lane + 64 * i;
        const int cc = c < C ? c : 0;     // chunks past the row end re-read chunk 0 (zero activations)
        vw[i] = cc * 16;
        lgrp[i] = group_of(cc << 5, gshift);
    }
    const int sz_first = row_begin * G;
    const int sz_al = sz_first & ~7;
    const int sz_pieces = ((row_end - row_begin) * G + (sz_first - sz_al) + 7) >> 3;
    const int szrow0 = sz_first - sz_al;               // LDS word of (row_begin, group 0)

    // 1. Issue order = need order (vmcnt waits are in issue order): activation staging
    //    loads, scale / zero staging loads, then the first weight batches.  All loads
    //    unconditional.
    u32x4 xv[JPT];
#pragma unroll
    for (int j = 0; j < JPT; ++j) {
        const int job = min(tid + NT * j, JOBS - 1);
        const int m = job / (CH * 4);
        const int e = job % (CH * 4);                  // 8-column block within the padded row
        const int c = e >> 2;
        xv[j] = reinterpret_cast<const u32x4*>(X + (size_t)m * K + ((size_t)(c < C ? c : 0) << 5))[e & 3];
    }
    //    Only waves that own staging pieces load them (wave-uniform branches): every vector
    //    memory instruction of the prologue delays the block's weight stream, redundant
    //    ones included (measured: 0.4 us per 7B-like step).
    u32x4 sv[JSZ], zv[JSZ];
#pragma unroll
    for (int j = 0; j < JSZ; ++j) {
        const int off = (sz_al + 8 * min(tid + NT * j, sz_pieces - 1)) * 2;
        if ((wave + W * j) * 64 < sz_pieces) {
            sv[j] = __builtin_amdgcn_raw_buffer_load_b128(src.s, off, 0, 0);
            zv[j] = __builtin_amdgcn_raw_buffer_load_b128(src.z, off, 0, 0);
        } else {
            sv[j] = u32x4{0u, 0u, 0u, 0u};
            zv[j] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    const int tail = min(full_end + (tid & 7), total - 1);
    const uint16_t st = __builtin_amdgcn_raw_buffer_load_b16(s_all, tail * 2, 0, 0);
    const uint16_t zt = __builtin_amdgcn_raw_buffer_load_b16(z_all, tail * 2, 0, 0);
    RowBatch<DT, M, CPL, RB> buf[NBUF];
#pragma unroll
    for (int i = 0; i < NBUF; ++i)
        load_batch<DT, M, CPL, RB, ONE>(buf[i], src, first + i * W * RB, nbatch > i, ONE ? wave_end : N, vw);
    __builtin_amdgcn_sched_barrier(0);

    // 2. Stage activations: permute each 8-column block, chunk sums by a quad reduction
    //    (the four blocks of a chunk sit in four consecutive lanes).  Branch-free except
    //    the predicated sum store; threads without a job write the spare slot.
#pragma unroll
    for (int j = 0; j < JPT; ++j) {
        const int job0 = tid + NT * j;
        const bool real = job0 < JOBS;
        const int job = real ? job0 : JOBS;            // spare: the slot past the last plane
        const int e = job % (CH * 4);
        const bool ok = real && (e >> 2) < C;
        const u32x4 v = xv[j];
        uint32_t o[4];
        if constexpr (DT == DT_F16)
            permute_x8(v.x, v.y, v.z, v.w, o);
        else
            permute_x8_byte(v.x, v.y, v.z, v.w, o);
        const uint32_t ones = DT == DT_F16 ? 0x3C003C00u : 0x3F803F80u;
        float sum = dot2<DT>(v.x, ones, 0.0f);
        sum = dot2<DT>(v.y, ones, sum);
        sum = dot2<DT>(v.z, ones, sum);
        sum = dot2<DT>(v.w, ones, sum);
        sum += dpp_mov<0xB1>(sum);                     // quad_perm [1,0,3,2]
        sum += dpp_mov<0x4E>(sum);                     // quad_perm [2,3,0,1]
        const int slot = real ? job >> 2 : M * CH;
        const int mrow = job / (CH * 4);
        const int piece_major = (mrow * 4 + (e & 3)) * PS + (e >> 2);
        reinterpret_cast<u32x4*>(xp)[real ? piece_major : 4 * M * PS] =
            ok ? u32x4{o[0], o[1], o[2], o[3]} : u32x4{0u, 0u, 0u, 0u};
        if ((job0 & 3) == 0)
            xsum[slot] = ok ? (DT == DT_F16 ? sum * 5.9604644775390625e-8f : sum) : 0.0f;
    }
    //    Group factors (s', c) per (row, group), see compute_batch; NULL zeros mean z = 8.
    auto factors = [&](uint32_t s_bits, uint32_t z_bits) {
        const float sv = h2f((uint16_t)s_bits);
        const float zv = has_zeros ? h2f((uint16_t)z_bits) : 8.0f;
        const float sp = DT == DT_F16 ? sv * 16777216.0f : sv;
        return float2{sp, -(DT == DT_F16 ? zv : 128.0f + zv) * sp};
    };
#pragma unroll
    for (int j = 0; j < JSZ; ++j) {
        const int p = tid + NT * j;
        if (p < sz_pieces && sz_al + 8 * p + 8 <= total) {
            const uint32_t sw[4] = {sv[j].x, sv[j].y, sv[j].z, sv[j].w};
            const uint32_t zw[4] = {zv[j].x, zv[j].y, zv[j].z, zv[j].w};
            float2* dst = szs + 8 * p;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                dst[2 * d] = factors(sw[d] & 0xFFFFu, zw[d] & 0xFFFFu);
                dst[2 * d + 1] = factors(sw[d] >> 16, zw[d] >> 16);
            }
        }
    }
    {
        const int h = full_end + tid;            // tail half of this thread (tid < 8)
        if (tid < 8 && h < total && h >= sz_al && h < sz_al + 8 * sz_pieces)
            szs[h - sz_al] = factors(st, zt);
    }
    __syncthreads();

    // 3. Row batches, NB in flight.  Prefetches are unconditional (a batch past the end
    //    loads zeros through `none`): a conditional prefetch would turn each buffer into a
    //    merge of old and new values and the compiler would shuffle registers, waiting on
    //    every load to do so.  The main loop runs while another round follows; the last
    //    round (the tail) only computes what is in flight, so a wave issues at most NB - 1
    //    empty batches.
    float acc[RB][M];
    if constexpr (ONE) {
        // all loads are in flight; compute in load order so each chunk waits only for itself
        if (nbatch > 0) {
            compute_batch<DT, M, CPL, RB>(buf[0], xp, xsum, szs, szrow0 + (first - row_begin) * G, G,
                                          wave_end - first, lgrp, C, gshift, lane, acc);
            store_batch<DT, M, RB>(acc, first, wave_end, N, lane, Y);
        }
    } else {
        int b = 0;
        for (; b + NB < nbatch; b += NB) {
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int row = first + (b + i) * W * RB;
                compute_batch<DT, M, CPL, RB>(buf[i], xp, xsum, szs, szrow0 + (row - row_begin) * G, G,
                                              row_end - row, lgrp, C, gshift, lane, acc);
                load_batch<DT, M, CPL, RB, false>(buf[i], src, first + (b + i + NB) * W * RB,
                                                  b + i + NB < nbatch, N, vw);
                store_batch<DT, M, RB>(acc, row, row_end, N, lane, Y);
            }
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            if (b + i < nbatch) {
                const int row = first + (b + i) * W * RB;
                compute_batch<DT, M, CPL, RB>(buf[i], xp, xsum, szs, szrow0 + (row - row_begin) * G, G,
                                              row_end - row, lgrp, C, gshift, lane, acc);
                store_batch<DT, M, RB>(acc, row, row_end, N, lane, Y);
            }
        }
    }
}

template <int DT, int M, int CPL, int RB, int W, int NB>
__global__ __launch_bounds__(64 * W) void gemv_stream_kernel(
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int has_zeros,
    uint16_t* __restrict__ Y, int N, int K, int G, int gshift, int rows_per_block) {
    extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
    stream_block<DT, M, CPL, RB, W, NB, kSzPiecesPerThread>(lds, X, qw, scales, zeros, has_zeros, Y, N, K, G,
                                                            gshift, rows_per_block, blockIdx.x);
}

struct GemvCfg {
    int nt = 0;
    int cpl = 0;
    int rb = 0;
};

constexpr int kMaxM = 8;
constexpr int cpl_max(int M) { return M == 1 ? 4 : (M == 2 ? 2 : 1); }

// Choose chunks-per-thread (best lane utilisation, then more chunks per thread) and
// rows-per-block (most rows that still give >= 2048 waves, i.e. 8 per CU; else 2).
GemvCfg pick(int M, int N, int K) {
    const int C = K / 32;
    GemvCfg best;
    double best_util = -1.0;
    for (int cpl = 1; cpl <= cpl_max(M); ++cpl) {
        const int nt = ((C + cpl - 1) / cpl + 63) / 64 * 64;
        if (nt > 1024 || nt > launch_limit(M, cpl, 2)) continue;
        const double util = (double)C / ((double)nt * cpl);
        if (util > best_util + 1e-9 || (util > best_util - 1e-9 && cpl > best.cpl)) {
            best_util = util;
            best.nt = nt;
            best.cpl = cpl;
        }
    }
    if (best.nt == 0) return best;
    const int waves_per_block = best.nt / 64;
    int rb = 2;
    for (int cand : {8, 4}) {
        const long long waves = (long long)((N + cand - 1) / cand) * waves_per_block;
        if (waves >= 2048 && best.nt <= launch_limit(M, best.cpl, cand)) {
            rb = cand;
            break;
        }
    }
    best.rb = rb;
    return best;
}

template <int DT, int M, int CPL, int RB>
hipError_t run3(const LinearArgs& a, int nt, hipStream_t st) {
    if constexpr (launch_limit(M, CPL, RB) == 0) {
        return hipErrorInvalidValue;
    } else {
        const int blocks = (a.N + RB - 1) / RB;
        hipLaunchKernelGGL((gemv_kernel<DT, M, CPL, RB>), dim3(blocks), dim3(nt), 0, st,
                           static_cast<const uint16_t*>(a.X), a.qw, a.scales, a.zeros,
                           a.zeros ? 1 : 0, static_cast<uint16_t*>(a.Y), a.N, a.K, a.G, a.gshift);
        return hipGetLastError();
    }
}

template <int DT, int M, int CPL>
hipError_t run2(const LinearArgs& a, const GemvCfg& c, hipStream_t st) {
    switch (c.rb) {
        case 2: return run3<DT, M, CPL, 2>(a, c.nt, st);
        case 4: return run3<DT, M, CPL, 4>(a, c.nt, st);
        case 8: return run3<DT, M, CPL, 8>(a, c.nt, st);
    }
    return hipErrorInvalidValue;
}

template <int DT, int M>
hipError_t run_m(const LinearArgs& a, const GemvCfg& c, hipStream_t st) {
    switch (c.cpl) {
        case 1: return run2<DT, M, 1>(a, c, st);
        case 2: if constexpr (cpl_max(M) >= 2) return run2<DT, M, 2>(a, c, st); break;
        case 3: if constexpr (cpl_max(M) >= 3) return run2<DT, M, 3>(a, c, st); break;
        case 4: if constexpr (cpl_max(M) >= 4) return run2<DT, M, 4>(a, c, st); break;
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

// Rows per batch of the streaming variant: two rows while a row is short, one row once
// a lane streams >= 4 chunks per row (two batches are in flight per wave).
constexpr int lds_rb(int M, int CPL) { return M * CPL >= 4 ? 1 : 2; }
// One-row layers up to K = 28672 (14 chunks per lane): the block stages the whole activation
// row (2 bytes per column plus a 4-byte sum per 32 columns) and its rows' group factors,
// 75 KB at K = 28672, so two blocks still share a CU's 160 KB of LDS.
constexpr int lds_max_cpl(int M) {
    return M == 1 ? 14 : (M == 2 ? 4 : (M == 3 ? 3 : (M == 4 ? 2 : 0)));
}
constexpr int kStreamLdsBudget = 80 * 1024;
constexpr int kDefaultLdsLimit = 64 * 1024;     // dynamic LDS above this must be requested
#ifndef W4A16_STREAM_WAVES
#define W4A16_STREAM_WAVES 8
#endif
#ifndef W4A16_ONE_ROW_BLOCKS
#define W4A16_ONE_ROW_BLOCKS 512
#endif
#ifndef W4A16_TWO_ROW_BLOCKS
#define W4A16_TWO_ROW_BLOCKS 768
#endif
constexpr int kPersistBlocks = 256;                    // one CU-resident block per CU
constexpr int kStreamBatches = 2;                      // row batches in flight per wave
constexpr int kStreamWaves = W4A16_STREAM_WAVES;       // waves per block: two per SIMD

struct LdsCfg {
    int cpl = 0;
    int blocks = 0;
    int rows_per_block = 0;
    int lds = 0;               // dynamic LDS bytes
};

// Rows per block: one row per wave while that takes at most kOneRowBlocks blocks (two per
// CU), else two rows per wave while that takes at most kTwoRowBlocks (three per CU), so the
// wave loads its rows at once; larger N: one block per CU (256), each owning ceil(N / 256)
// rows streamed in batches.  One-row layers whose rows give a lane >= 4 chunks always take
// one row per wave, loaded at once, in as many blocks as that needs: the hardware keeps
// several such blocks per CU in flight and refills the CU as they end, which streams faster
// than a CU-resident block walking its rows in batches (measured on 8192 -> 28672:
// 21.9 us against 24.6 us, 8192 -> 8192: 8.0 against 8.4 us).  The block's activations,
// chunk sums and (scale, zero) words must fit the LDS budget.
constexpr int kOneRowBlocks = W4A16_ONE_ROW_BLOCKS;
constexpr int kTwoRowBlocks = W4A16_TWO_ROW_BLOCKS;
LdsCfg pick_lds(int M, int N, int K, int G) {
    LdsCfg c;
    if (M < 1 || M > 4) return c;
    const int cpl = (K / 32 + 63) / 64;
    if (cpl > lds_max_cpl(M)) return c;
    // 32-bit buffer offsets: the packed weights must stay below 2 GiB
    if ((long long)N * (K / 2) >= (1LL << 31)) return c;
    int rpb = (N + kPersistBlocks - 1) / kPersistBlocks;
    if ((M == 1 && cpl >= 4) || (N + kStreamWaves - 1) / kStreamWaves <= kOneRowBlocks)
        rpb = kStreamWaves;
    else if ((N + 2 * kStreamWaves - 1) / (2 * kStreamWaves) <= kTwoRowBlocks)
        rpb = 2 * kStreamWaves;
    const long long pieces = ((long long)rpb * G + 7) / 8 + 1;      // 16-byte staging pieces
    if (pieces > (long long)kSzPiecesPerThread * 64 * kStreamWaves) return c;
    const long long lds = sz_lds_offset(M, cpl) + 64 * pieces;       // 8 float pairs per piece
    if (lds > kStreamLdsBudget) return c;
    c.cpl = cpl;
    c.rows_per_block = rpb;
    c.blocks = (N + rpb - 1) / rpb;
    c.lds = (int)lds;
    return c;
}

// When a wave owns at most two rows and they fit in registers (at most kOneShotLoads
// 16-byte loads per lane), the wave loads all of them at once (NB = 0, one batch);
// otherwise batches of lds_rb rows, two in flight (measured faster for longer row runs).
constexpr int kOneShotLoads = 12;
constexpr int kOneShotRows = 2;
template <int DT, int M, int CPL, int RB, int NB>
hipError_t run_lds4(const LinearArgs& a, const LdsCfg& c, hipStream_t st) {
    if (c.lds > kDefaultLdsLimit) {
        const hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&gemv_stream_kernel<DT, M, CPL, RB, kStreamWaves, NB>),
            hipFuncAttributeMaxDynamicSharedMemorySize, c.lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((gemv_stream_kernel<DT, M, CPL, RB, kStreamWaves, NB>), dim3(c.blocks),
                       dim3(64 * kStreamWaves), c.lds, st,
                       static_cast<const uint16_t*>(a.X), a.qw, a.scales, a.zeros, a.zeros ? 1 : 0,
                       static_cast<uint16_t*>(a.Y), a.N, a.K, a.G, a.gshift, c.rows_per_block);
    return hipGetLastError();
}

template <int DT, int M, int CPL, int RB>
hipError_t run_one(const LinearArgs& a, const LdsCfg& c, hipStream_t st) {
    if constexpr (M == 1 && CPL >= 4) {
        // one row per wave, loaded at once (pick_lds)
        if (c.rows_per_block != kStreamWaves) return hipErrorInvalidValue;
        return run_lds4<DT, 1, CPL, 1, 0>(a, c, st);
    } else if constexpr (RB > kOneShotRows || RB * M * CPL > kOneShotLoads) {
        return run_lds4<DT, M, CPL, lds_rb(M, CPL), kStreamBatches>(a, c, st);
    } else {
        if (c.rows_per_block <= RB * kStreamWaves) return run_lds4<DT, M, CPL, RB, 0>(a, c, st);
        return run_one<DT, M, CPL, RB + 1>(a, c, st);
    }
}

template <int DT, int M, int CPL>
hipError_t run_lds3(const LinearArgs& a, const LdsCfg& c, hipStream_t st) {
    return run_one<DT, M, CPL, 1>(a, c, st);
}

template <int DT, int M, int CPL>
hipError_t run_lds_cpl(const LinearArgs& a, const LdsCfg& c, hipStream_t st) {
    if constexpr (CPL > lds_max_cpl(M)) {
        return hipErrorInvalidValue;
    } else {
        if (c.cpl == CPL) return run_lds3<DT, M, CPL>(a, c, st);
        return run_lds_cpl<DT, M, CPL + 1>(a, c, st);
    }
}

template <int DT>
hipError_t run_lds(const LinearArgs& a, const LdsCfg& c, hipStream_t st) {
    switch (a.M) {
        case 1: return run_lds_cpl<DT, 1, 1>(a, c, st);
        case 2: return run_lds_cpl<DT, 2, 1>(a, c, st);
        case 3: return run_lds_cpl<DT, 3, 1>(a, c, st);
        case 4: return run_lds_cpl<DT, 4, 1>(a, c, st);
    }
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------------
// Grouped launch: several independent one-row layers (M = 1) in one kernel.  Each launch
// pays a fixed cost of about 1.8 us on this GPU (dispatch behind the previous kernel, ramp
// up, drain), which at decode is comparable to streaming a whole 7B-sized layer; one grid
// over the layers pays it once.  Block b works for the layer whose block range holds b and
// runs the streaming block body for that layer, so every output is computed exactly as by
// the layer's own launch (same lane-to-chunk mapping, same order of sums).
//
// The kernel is bound by the weight bytes a CU keeps in flight: a wave's loads are all
// issued at its start and its registers hold them until it has computed, so the rate
// follows the number of resident waves.  Every variant of the switch below shares one
// register allocation, the largest; the variants are chosen so that it stays at 64 VGPRs,
// which lets 8 waves share a SIMD: two rows per wave for up to 2 chunks per lane
// (K <= 4096), one row for 3 .. 6 chunks (K <= 12288; two rows at 3 chunks took 79 VGPRs).
// Blocks of 8 waves stage the activations once for twice the rows of 4-wave blocks, and each
// thread stages at most one 16-byte piece of scales and one of zeros.  Measured on the
// 7B-like step (4096 x 4096, 4096 -> 11008, 11008 -> 4096), 200 launches per graph replay:
// 4-wave blocks at 89 VGPRs (5 waves per SIMD) 14.3 us; 8-wave blocks at 82 VGPRs 14.3 us;
// the same capped at 80 VGPRs (6 per SIMD, two registers spilled) 12.6-12.8 us; this form
// (64 VGPRs, 8 per SIMD, no spills) 12.5 us; a plain read of the same 56.8 MB in one
// launch takes 9.9 us at best.
constexpr int kGroupMax = 16;
constexpr int kGroupWaves = 8;        // waves per block of the grouped kernel
constexpr int kGroupSzPieces = 1;     // staged 16-byte scale (and zero) pieces per thread
constexpr int kGroupMaxCpl = 6;       // chunks per lane of the kernel's variants (K <= 12288)
constexpr int group_rows_per_wave(int cpl) { return cpl <= 2 ? 2 : 1; }

struct GroupItem {
    const uint16_t* X;
    const uint32_t* qw;
    const uint16_t* scales;
    const uint16_t* zeros;
    uint16_t* Y;
    int N, K, G, gshift;
    int rows_per_block;
    int block_begin;       // first grid block of this layer
    int variant;           // chunks per lane: the case of the kernel's switch
    int has_zeros;
};

struct GroupArgs {
    GroupItem it[kGroupMax];
    int count;
};


template <int DT>
__global__ __launch_bounds__(64 * kGroupWaves) void gemv_group_kernel(const GroupArgs ga) {
    extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
    const int b = blockIdx.x;
    int i = 0;
#pragma unroll
    for (int j = 1; j < kGroupMax; ++j)
        if (j < ga.count && b >= ga.it[j].block_begin) i = j;
    const GroupItem& t = ga.it[i];
    const int lb = b - t.block_begin;
#define W4A16_GROUP_CASE(CPL)                                                                             \
    case CPL:                                                                                          \
        stream_block<DT, 1, CPL, group_rows_per_wave(CPL), kGroupWaves, 0, kGroupSzPieces>(              \
            lds, t.X, t.qw, t.scales, t.zeros, t.has_zeros, t.Y, t.N, t.K, t.G, t.gshift, t.rows_per_block, lb); \
        break;
    switch (t.variant) {
        W4A16_GROUP_CASE(1)
        W4A16_GROUP_CASE(2)
        W4A16_GROUP_CASE(3)
        W4A16_GROUP_CASE(4)
        W4A16_GROUP_CASE(5)
        W4A16_GROUP_CASE(6)
        default: break;
    }
#undef W4A16_GROUP_CASE
}

// The grouped configuration of one layer, or cpl == 0 if the grouped kernel cannot take it.
LdsCfg pick_group(const LinearArgs& a, int* rb) {
    LdsCfg c;
    if (a.M != 1) return c;
    const int cpl = (a.K / 32 + 63) / 64;
    if (cpl > kGroupMaxCpl) return c;
    if ((long long)a.N * (a.K / 2) >= (1LL << 31)) return c;
    *rb = group_rows_per_wave(cpl);
    const int rpb = *rb * kGroupWaves;
    const long long pieces = ((long long)rpb * a.G + 7) / 8 + 1;
    if (pieces > (long long)kGroupSzPieces * 64 * kGroupWaves) return c;
    const long long lds = sz_lds_offset(1, cpl) + 64 * pieces;
    if (lds > kLdsBudget) return c;
    c.cpl = cpl;
    c.rows_per_block = rpb;
    c.blocks = (a.N + rpb - 1) / rpb;
    c.lds = (int)lds;
    return c;
}

}  // namespace

bool gemv_group_supports(const LinearArgs& a) {
    int rb = 0;
    return pick_group(a, &rb).cpl > 0;
}

hipError_t launch_gemv_group(const LinearArgs* items, int count, hipStream_t st) {
    if (count < 1 || count > kGroupMax) return hipErrorInvalidValue;
    GroupArgs ga{};
    ga.count = count;
    long long blocks = 0;
    int lds = 0;
    // blocks of the layers with the longest rows (the longest-lived blocks) are dispatched first
    int order[kGroupMax];
    for (int i = 0; i < count; ++i) order[i] = i;
    std::stable_sort(order, order + count, [&](int x, int y) { return items[x].K > items[y].K; });
    for (int oi = 0; oi < count; ++oi) {
        const int i = oi;
        const LinearArgs& a = items[order[oi]];
        if (a.dtype != items[0].dtype) return hipErrorInvalidValue;
        int rb = 0;
        const LdsCfg c = pick_group(a, &rb);
        if (c.cpl == 0) return hipErrorInvalidValue;
        GroupItem& t = ga.it[i];
        t.X = static_cast<const uint16_t*>(a.X);
        t.qw = a.qw;
        t.scales = a.scales;
        t.zeros = a.zeros;
        t.Y = static_cast<uint16_t*>(a.Y);
        t.N = a.N;
        t.K = a.K;
        t.G = a.G;
        t.gshift = a.gshift;
        t.rows_per_block = c.rows_per_block;
        t.block_begin = (int)blocks;
        t.variant = c.cpl;
        t.has_zeros = a.zeros ? 1 : 0;
        blocks += c.blocks;
        lds = lds > c.lds ? lds : c.lds;
    }
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (items[0].dtype == DT_F16)
        hipLaunchKernelGGL(gemv_group_kernel<DT_F16>, dim3((unsigned)blocks), dim3(64 * kGroupWaves), lds, st, ga);
    else
        hipLaunchKernelGGL(gemv_group_kernel<DT_BF16>, dim3((unsigned)blocks), dim3(64 * kGroupWaves), lds, st, ga);
    return hipGetLastError();
}

bool gemv_supports(const LinearArgs& a) {
    if (a.M < 1 || a.M > kMaxM) return false;
    return pick_lds(a.M, a.N, a.K, a.G).cpl > 0 || pick(a.M, a.N, a.K).nt > 0;
}

hipError_t launch_gemv(const LinearArgs& a, hipStream_t st) {
    const LdsCfg lc = pick_lds(a.M, a.N, a.K, a.G);
    if (lc.cpl > 0)
        return a.dtype == DT_F16 ? run_lds<DT_F16>(a, lc, st) : run_lds<DT_BF16>(a, lc, st);
    const GemvCfg c = pick(a.M, a.N, a.K);
    if (c.nt == 0) return hipErrorInvalidValue;
    return a.dtype == DT_F16 ? run_dt<DT_F16>(a, c, st) : run_dt<DT_BF16>(a, c, st);
}

}  // namespace w4a16
