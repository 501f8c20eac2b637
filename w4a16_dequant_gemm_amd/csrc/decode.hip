// Decode-regime W4A16 kernels on CDNA4 matrix cores, 1 <= M <= 16 (MFMA 16x16x32);
// K % 256 == 0 and g % 128 == 0.  decode_kernel (M <= 4) stages the activations in LDS;
// decode_ring_kernel (M <= 16; used from 5 rows, or when the activations do not fit the LDS)
// loads them from memory next to a weight stream that goes straight into an LDS ring.
//
// At decode the layer streams every packed weight once per token (page
// "推理优化中“用精度换性能“的核心技术：量化", section 一), so the kernel is built around the
// HBM stream; the arithmetic has to stay cheap enough to hide behind it.  A VALU dot
// product spends about 13 vector instructions per packed 32-bit word (unpack, four
// v_dot2, the per-chunk scale and the per-row cross-lane sum); here the matrix cores take
// the multiply-adds and the k-reduction, and the VALU only unpacks (five instructions per
// word) and folds one scale per (16-row tile, k-block).  Dequantization stays in registers
// (page "大模型推理中 Weight-only、W8A8 和 FP8 量化有什么区别？如何选型？", section 二).
//
// Work split.  A block of W waves owns up to T consecutive 16-row tiles and all of K; wave
// w takes the k-block pairs (256 columns) kp0 .. kp1-1 and visits every tile of the block
// for each of them, keeping P pairs of weight loads in flight.  The waves' partial tiles
// are summed in LDS at the end.
//
// Weight stream.  The unit of loading is (tile, k-block pair): 16 rows x 128 bytes, two
// 16-byte loads per lane, load h giving lane l row 8 h + l / 8, bytes 16 (l % 8) .. +15 of
// the pair.  Every eight consecutive lanes read 128 contiguous bytes, a full cache line,
// so an instruction makes eight line requests.  The MFMA B operand needs another
// assignment (lane L: row L % 16, 16-byte piece L / 16 of the k-block), so each unit goes
// through a per-wave 2 KB LDS buffer: (row r, piece c) lives in slot 8 r + (c ^ (r / 2 % 8)),
// which keeps both the writes and the reads free of bank conflicts.
//
// Operands (lane L: n = L % 16, q = L / 16; MFMA j of a k-block takes word j of the
// piece, columns 128 kb + 32 q + 8 j .. +7).
//   fp16 weights: mask unpack, five instructions per word, registers (u0,u4) (16u1,16u5)
//     (u2,u6) (16u3,16u7) as fp16 subnormals times 2^-24 (the matrix cores multiply
//     subnormals exactly).  The activation fragment is staged in the same order with the
//     x16 slots' activations divided by 16, so every product is x * u * 2^-24; the division
//     is exact unless |x| < 2^-10, where it rounds to a multiple of 2^-24 (an absolute
//     error below 2^-25 in x / 16).
//   bf16 weights: byte unpack to 128 + u, activations in the matching byte order.
//   Activations: the wave's slice of X sits in LDS; all lanes of a 16-lane row read the
//     same activation row (rows m >= M repeat row M - 1), so the reads broadcast and the
//     extra accumulator rows only duplicate real ones.
//   Zero point and scale: tile += s' * (acc - c * S) per (tile, k-block), S the k-block's
//     activation sum (staging pass, 16-lane DPP sum); fp16: s' = s * 2^24, c = z;
//     bf16: s' = s, c = 128 + z.  (scale, zero) pairs of the block's rows are staged in
//     LDS with coalesced loads, one 32-bit word per (row, group).
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace w4a16 {

namespace {

constexpr int kWaves = 8;
constexpr int kLdsBudget = 65536;
constexpr int kSzPieces = 2;           // 16-byte scale (and zero) staging pieces per thread

__host__ __device__ constexpr int align16(int v) { return (v + 15) & ~15; }

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

template <int T>
struct Stage {
    u32x4 w[T][2];
};

template <int T>
__device__ __forceinline__ void load_stage(Stage<T>& st, __amdgpu_buffer_rsrc_t w, __amdgpu_buffer_rsrc_t none,
                                           int kp, bool live, const int vw[T][2], int ntiles) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const __amdgpu_buffer_rsrc_t r = live && t < ntiles ? w : none;   // wave-uniform
#pragma unroll
        for (int h = 0; h < 2; ++h)
            st.w[t][h] = __builtin_amdgcn_raw_buffer_load_b128(r, vw[t][h], kp * 128, 2 /* nt */);
    }
}

// One k-block pair for the block's T tiles.
template <int DT, int M, int T>
__device__ __forceinline__ void compute_kp(const Stage<T>& st, u32x4* wt, const int wslot[2],
                                           const int rslot[2], const uint16_t* xa, const float* sk,
                                           const int sidx[M], const uint32_t* szl, const int szo[T],
                                           int kp, int gshift, f32x4 tile[T]) {
    uint32_t a[2][4][4];
    float S[2][M];
    int grp[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int kb = 2 * kp + e;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(xa + kb * 128 + 8 * j);
            a[e][j][0] = v.x; a[e][j][1] = v.y; a[e][j][2] = v.z; a[e][j][3] = v.w;
        }
#pragma unroll
        for (int j = 0; j < M; ++j) S[e][j] = sk[kb * 4 + sidx[j]];
        grp[e] = (kb << 7) >> gshift;
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
        // transpose the unit through the wave's LDS slots (LDS requests of a wave run in
        // order, so the next tile's writes cannot overtake these reads)
        wt[wslot[0]] = st.w[t][0];
        wt[wslot[1]] = st.w[t][1];
        __builtin_amdgcn_wave_barrier();
        u32x4 wb[2];
        wb[0] = wt[rslot[0]];
        wb[1] = wt[rslot[1]];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            uint32_t b[4][4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (DT == DT_F16)
                    unpack_mask_f16(wb[e][j], b[j]);
                else
                    unpack_byte<0x43>(wb[e][j], b[j]);
            }
            f32x4 acc = mfma16<DT>(a[e][0], b[0], f32x4{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
            for (int j = 1; j < 4; ++j) acc = mfma16<DT>(a[e][j], b[j], acc);
            const uint32_t sz = szl[szo[t] + grp[e]];
            const float s = h2f((uint16_t)(sz & 0xFFFFu));
            const float z = h2f((uint16_t)(sz >> 16));
            const float sp = DT == DT_F16 ? s * 16777216.0f : s;
            const float c = DT == DT_F16 ? z : 128.0f + z;
#pragma unroll
            for (int j = 0; j < M; ++j) tile[t][j] = fmaf(sp, fmaf(-c, S[e][j], acc[j]), tile[t][j]);
        }
    }
}

template <int DT, int M, int T, int P, int W>
__global__ __launch_bounds__(64 * W) void decode_kernel(
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int has_zeros,
    uint16_t* __restrict__ Y, int N, int K, int G, int gshift, int NT, int nblk, int KSP,
    int off_sk, int off_spare, int off_szs, int off_wt) {
    extern __shared__ __attribute__((aligned(16))) uint32_t dlds[];
    constexpr int NTH = 64 * W;
    const int KB = K >> 7;
    const int xpitch = KB * 128 + 8;             // halves per LDS activation row (16 B pad)
    unsigned char* lbase = reinterpret_cast<unsigned char*>(dlds);
    uint16_t* xs = reinterpret_cast<uint16_t*>(lbase);
    float* sk = reinterpret_cast<float*>(lbase + off_sk);                 // [KB][4]
    uint16_t* xspare = reinterpret_cast<uint16_t*>(lbase + off_spare);
    float* sspare = reinterpret_cast<float*>(lbase + off_spare + 16);
    uint32_t* szs = reinterpret_cast<uint32_t*>(lbase + off_szs);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    u32x4* wt = reinterpret_cast<u32x4*>(lbase + off_wt) + wave * 128;     // 2 KB per wave
    const int n16 = lane & 15;
    const int q = lane >> 4;

    // tiles of this block: an even split of the NT tiles over the grid
    const int tile0 = (int)(((long long)blockIdx.x * NT) / nblk);
    const int ntiles = (int)(((long long)(blockIdx.x + 1) * NT) / nblk) - tile0;
    const int row_begin = tile0 * 16;
    const int row_end = min(N, row_begin + ntiles * 16);
    const int kp0 = wave * KSP;                      // k-block pairs of this wave
    const int kp1 = min(KB / 2, kp0 + KSP);
    const int np = max(0, kp1 - kp0);
    const int kb0 = 2 * kp0;
    const int nk = 2 * np;                           // k-blocks of this wave

    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(qw), 0, 0x7FFFFFFF, 0x00020000);
    const __amdgpu_buffer_rsrc_t none =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(qw), 0, 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(X), 0, M * K * 2, 0x00020000);
    // scales / zeros (NULL zeros read the scales, replaced by 8): 16-byte pieces that lie
    // wholly inside the arrays, plus the last (N * G) % 8 halves with 2-byte loads
    const uint16_t* zsrc = has_zeros ? zeros : scales;
    const int total = N * G;
    const int full_end = total & ~7;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(scales), 0, full_end * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rz =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(zsrc), 0, full_end * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_all =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(scales), 0, total * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rz_all =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(zsrc), 0, total * 2, 0x00020000);

    // weight load mapping: load h, lane l -> row 8 h + l / 8, piece l % 8 of the unit;
    // LDS slot of (row r, piece c): 8 r + (c ^ (r / 2 % 8))
    int vw[T][2], wslot[2], rslot[2];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int n = min((tile0 + t) * 16 + 8 * h + (lane >> 3), N - 1);   // rows past N: clamped
            vw[t][h] = n * (K >> 1) + 16 * (lane & 7);
        }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = 8 * h + (lane >> 3);
        wslot[h] = 8 * r + ((lane & 7) ^ ((r >> 1) & 7));
        const int c = 4 * h + q;                      // piece of k-block 2 kp + h
        rslot[h] = 8 * n16 + (c ^ ((n16 >> 1) & 7));
    }

    // 1. Loads in need order (vmcnt waits are in issue order): activation pieces of the
    //    wave's slice, the block's scales and zeros, then P k-blocks of weights.
    //    Activation piece p (8 columns): row p / (16 nk), column 128 kb0 + 8 (p % (16 nk)).
    constexpr int JX = 4;
    const int per_row = nk * 16;
    const int npieces = M * per_row;
    auto x_row = [&](int p) {
        int m = 0;
#pragma unroll
        for (int r = 1; r < M; ++r) m += p >= r * per_row ? 1 : 0;
        return m;
    };
    auto x_off = [&](int p) {
        p = min(p, max(npieces - 1, 0));
        const int m = x_row(p);
        return (m * K + kb0 * 128 + 8 * (p - m * per_row)) * 2;
    };
    u32x4 xv[JX];
#pragma unroll
    for (int i = 0; i < JX; ++i)
        xv[i] = __builtin_amdgcn_raw_buffer_load_b128(nk > 0 ? rx : none, x_off(lane + 64 * i), 0, 0);
    const int sz_first = row_begin * G;
    const int sz_al = sz_first & ~7;
    const int sz_pieces = ((row_end - row_begin) * G + (sz_first - sz_al) + 7) >> 3;
    // only waves that own staging pieces load them (wave-uniform): redundant prologue loads
    // delay the weight stream
    u32x4 sv[kSzPieces], zv[kSzPieces];
#pragma unroll
    for (int j = 0; j < kSzPieces; ++j) {
        const int off = (sz_al + 8 * min(tid + NTH * j, sz_pieces - 1)) * 2;
        if ((wave + W * j) * 64 < sz_pieces) {
            sv[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
            zv[j] = __builtin_amdgcn_raw_buffer_load_b128(rz, off, 0, 0);
        } else {
            sv[j] = u32x4{0u, 0u, 0u, 0u};
            zv[j] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    const int tail = min(full_end + (tid & 7), total - 1);
    const uint16_t s_tail = __builtin_amdgcn_raw_buffer_load_b16(rs_all, tail * 2, 0, 0);
    const uint16_t z_tail = __builtin_amdgcn_raw_buffer_load_b16(rz_all, tail * 2, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    Stage<T> st[P];
#pragma unroll
    for (int p = 0; p < P; ++p) load_stage<T>(st[p], rw, none, kp0 + p, p < np, vw, ntiles);
    __builtin_amdgcn_sched_barrier(0);

    // 2. Staging, branch-free where a branch could pull the loads above behind it (a lane
    //    without a piece writes the spare slots).  Activations in the unpack's pair order
    //    (fp16: the x16 code slots divided by 16), k-block sums by a 16-lane DPP sum.
    const uint32_t ones = DT == DT_F16 ? 0x3C003C00u : 0x3F803F80u;
    auto stage_x = [&](const u32x4 (&v4)[JX], int base) {
#pragma unroll
        for (int i = 0; i < JX; ++i) {
            const int p = base + lane + 64 * i;
            const u32x4 v = v4[i];
            float sum = dot2<DT>(v.x, ones, 0.0f);
            sum = dot2<DT>(v.y, ones, sum);
            sum = dot2<DT>(v.z, ones, sum);
            sum = dot2<DT>(v.w, ones, sum);
            sum += dpp_mov<0xB1>(sum);       // quad_perm [1,0,3,2]
            sum += dpp_mov<0x4E>(sum);       // quad_perm [2,3,0,1]
            sum += dpp_mov<0x141>(sum);      // row_half_mirror
            sum += dpp_mov<0x140>(sum);      // row_mirror: 16-lane (one k-block) sum
            const bool ok = p < npieces;
            const int m = x_row(p);
            const int e = p - m * per_row;
            uint32_t o[4];
            if constexpr (DT == DT_F16) {
                permute_x8(v.x, v.y, v.z, v.w, o);
                const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
                o[1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, o[1]) * sixteenth);
                o[3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, o[3]) * sixteenth);
            } else {
                permute_x8_byte(v.x, v.y, v.z, v.w, o);
            }
            uint16_t* xd = ok ? xs + m * xpitch + kb0 * 128 + 8 * e : xspare;
            *reinterpret_cast<u32x4*>(xd) = u32x4{o[0], o[1], o[2], o[3]};
            float* sd = ok && (e & 15) == 0 ? sk + (kb0 + (e >> 4)) * 4 + m : sspare;
            *sd = DT == DT_F16 ? sum * 5.9604644775390625e-8f : sum;
        }
    };
    stage_x(xv, 0);
    //    (scale | zero << 16) words; NULL zeros become 8.0 (0x4800)
#pragma unroll
    for (int j = 0; j < kSzPieces; ++j) {
        const int p = tid + NTH * j;
        const u32x4 sw = sv[j];
        const u32x4 zw = has_zeros ? zv[j] : u32x4{0x48004800u, 0x48004800u, 0x48004800u, 0x48004800u};
        if (p < sz_pieces && sz_al + 8 * p + 8 <= total) {
            u32x4* dst = reinterpret_cast<u32x4*>(szs + 8 * p);
            dst[0] = u32x4{perm(zw.x, sw.x, 0x05040100u), perm(zw.x, sw.x, 0x07060302u),
                           perm(zw.y, sw.y, 0x05040100u), perm(zw.y, sw.y, 0x07060302u)};
            dst[1] = u32x4{perm(zw.z, sw.z, 0x05040100u), perm(zw.z, sw.z, 0x07060302u),
                           perm(zw.w, sw.w, 0x05040100u), perm(zw.w, sw.w, 0x07060302u)};
        }
    }
    {
        const int h = full_end + tid;            // tail half of this thread (tid < 8)
        if (tid < 8 && h < total && h >= sz_al && h < sz_al + 8 * sz_pieces)
            szs[h - sz_al] = (uint32_t)s_tail | ((uint32_t)(has_zeros ? z_tail : (uint16_t)0x4800) << 16);
    }
    for (int r = 1; r * 64 * JX < npieces; ++r) {     // long slices: more activation rounds
        u32x4 xr[JX];
#pragma unroll
        for (int i = 0; i < JX; ++i)
            xr[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, x_off(r * 64 * JX + lane + 64 * i), 0, 0);
        stage_x(xr, r * 64 * JX);
    }
    __syncthreads();

    // 3. k-blocks of the slice, P in flight.  The main loop runs while another round
    //    follows; the last round only computes what is in flight.
    const uint16_t* xa = xs + min(n16, M - 1) * xpitch + 32 * q;
    int sidx[M];
#pragma unroll
    for (int j = 0; j < M; ++j) sidx[j] = min(4 * q + j, M - 1);
    int szo[T];
#pragma unroll
    for (int t = 0; t < T; ++t) szo[t] = (sz_first - sz_al) + (t * 16 + n16) * G;
    f32x4 tile[T];
#pragma unroll
    for (int t = 0; t < T; ++t) tile[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    int i = 0;
    for (; i + P < np; i += P) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
            compute_kp<DT, M, T>(st[p], wt, wslot, rslot, xa, sk, sidx, szs, szo, kp0 + i + p, gshift, tile);
            load_stage<T>(st[p], rw, none, kp0 + i + p + P, i + p + P < np, vw, ntiles);
        }
    }
#pragma unroll
    for (int p = 0; p < P; ++p)
        if (i + p < np)
            compute_kp<DT, M, T>(st[p], wt, wslot, rslot, xa, sk, sidx, szs, szo, kp0 + i + p, gshift, tile);

    // 4. Sum the waves' partial tiles in the LDS (no longer used from offset 0);
    //    lane (n, q) element j is row 4 q + j.
    __syncthreads();
    f32x4* red = reinterpret_cast<f32x4*>(lbase);               // [W][T][64]
#pragma unroll
    for (int t = 0; t < T; ++t) red[(wave * T + t) * 64 + lane] = tile[t];
    __syncthreads();
    if (tid < T * 64) {
        const int t = tid >> 6;
        const int l = tid & 63;
        f32x4 v = red[t * 64 + l];
        for (int w = 1; w < W; ++w) {
            const f32x4 u = red[(w * T + t) * 64 + l];
            v[0] += u[0]; v[1] += u[1]; v[2] += u[2]; v[3] += u[3];
        }
        const int n = (tile0 + t) * 16 + (l & 15);
        if (t < ntiles && n < N) {
#pragma unroll
            for (int j = 0; j < M; ++j) {
                const int m = 4 * (l >> 4) + j;
                if (m < M) Y[(size_t)m * N + n] = f2out<DT>(v[j]);
            }
        }
    }
}

// Activation fragments of one k-block pair in registers (ring kernel): lane (n, q) holds row
// n, columns 128 kb + 32 q .. + 31 of each k-block of the pair.
struct XStage {
    u32x4 x[2][4];
};

// ---------------------------------------------------------------------------------
// Up to 16 rows (used from 5 rows, or when the activations do not fit decode_kernel's LDS),
// with the weight stream in an LDS ring.  Holding the weight loads in flight in registers,
// next to the activation fragments, caps a CU at about 32 KB of weights in flight (two waves
// per SIMD); the HBM stream needs several times that.  Here the weights go from memory
// straight into LDS (buffer loads with the LDS-direct form, no registers while in flight):
// each wave owns a ring of D = T * PK
// slots of one (tile, k-block pair) unit each, 2 KB, and refills a slot as soon as its
// unit is in registers, so PK k-block pairs of all T tiles are in flight per wave, up to
// 128 KB per CU.  Every slot is an LDS object of its own, so the compiler's waits on the
// loads name exactly the slot being read (one object for all slots would make every read
// wait for the whole ring).  The activations no longer fit the LDS (16 rows of K), so each
// wave loads the fragments of its k-block pairs straight from memory (L2-resident: every
// block reads all of X) into registers one pair ahead, where they serve all T tiles; lane
// (n, q) loads row n (zeros for n >= M) and puts it in the unpack's pair order.  The
// k-block activation sums come from four more MFMAs against a constant B operand (2^-24 in
// the x1 slots and 16 * 2^-24 in the x16 slots for fp16, 1.0 for bf16), so they land in
// the accumulator layout: lane (n, q) element j holds row 4 q + j.
//
// Unit layout in a slot: load instruction h (0, 1), lane l fetches row r = 8 h + l / 8 of
// the tile, 16-byte piece (l % 8) ^ (r / 2 % 8) of the pair's 128 bytes, and lands in slot
// word 64 h + l = 8 r + l % 8 (eight consecutive lanes still read one 128-byte line, only
// in permuted order); lane (n, q) later reads piece 4 e + q of row n (k-block e of the
// pair) from word 8 n + ((4 e + q) ^ (n / 2 % 8)), free of bank conflicts.  The MFMA
// operands and the per-(tile, k-block) scale fold are those of decode_kernel.
constexpr int kRingSlots = 8;
constexpr int kRingUnit = 128;              // 16-byte words per unit (2 KB)
__shared__ __attribute__((aligned(16))) u32x4 g_ring0[kWaves][kRingUnit];
__shared__ __attribute__((aligned(16))) u32x4 g_ring1[kWaves][kRingUnit];
__shared__ __attribute__((aligned(16))) u32x4 g_ring2[kWaves][kRingUnit];
__shared__ __attribute__((aligned(16))) u32x4 g_ring3[kWaves][kRingUnit];
__shared__ __attribute__((aligned(16))) u32x4 g_ring4[kWaves][kRingUnit];
__shared__ __attribute__((aligned(16))) u32x4 g_ring5[kWaves][kRingUnit];
__shared__ __attribute__((aligned(16))) u32x4 g_ring6[kWaves][kRingUnit];
__shared__ __attribute__((aligned(16))) u32x4 g_ring7[kWaves][kRingUnit];

template <int d>
__device__ __forceinline__ u32x4* ring_slot(int wave) {
    static_assert(d >= 0 && d < kRingSlots, "ring slot");
    if constexpr (d == 0) return g_ring0[wave];
    else if constexpr (d == 1) return g_ring1[wave];
    else if constexpr (d == 2) return g_ring2[wave];
    else if constexpr (d == 3) return g_ring3[wave];
    else if constexpr (d == 4) return g_ring4[wave];
    else if constexpr (d == 5) return g_ring5[wave];
    else if constexpr (d == 6) return g_ring6[wave];
    else return g_ring7[wave];
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Both load instructions of one unit into ring slot d.
template <int d>
__device__ __forceinline__ void ring_fill(__amdgpu_buffer_rsrc_t r, int wave, const int vw[2], int kp) {
    u32x4* s = ring_slot<d>(wave);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)s, 16, vw[0],
                                             kp * 128, 0, 2 /* nt */);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(s + 64), 16, vw[1],
                                             kp * 128, 0, 2 /* nt */);
}

// One block of the ring kernel: block `bid` of a layer's grid of `nblk` blocks (the
// single-layer kernel and the grouped kernel both run this body).
template <int DT, int T, int PK>
__device__ __forceinline__ void ring_block(
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int has_zeros,
    uint16_t* __restrict__ Y, int M, int N, int K, int G, int gshift, int NT, int nblk, int KSP, int bid) {
    constexpr int W = kWaves;
    constexpr int NTH = 64 * W;
    static_assert(T * PK <= kRingSlots && T <= W, "ring configuration");
    extern __shared__ __attribute__((aligned(16))) uint32_t dlds[];
    uint32_t* szs = dlds;                                                  // (s | z << 16) words
    const int KB = K >> 7;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15;
    const int q = lane >> 4;

    const int tile0 = (int)(((long long)bid * NT) / nblk);
    const int ntiles = (int)(((long long)(bid + 1) * NT) / nblk) - tile0;
    const int row_begin = tile0 * 16;
    const int row_end = min(N, row_begin + ntiles * 16);
    const int kp0 = wave * KSP;
    const int kp1 = min(KB / 2, kp0 + KSP);
    const int np = max(0, kp1 - kp0);

    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(qw), 0, 0x7FFFFFFF, 0x00020000);
    const __amdgpu_buffer_rsrc_t none =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(qw), 0, 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(X), 0, M * K * 2, 0x00020000);
    const uint16_t* zsrc = has_zeros ? zeros : scales;
    const int total = N * G;
    const int full_end = total & ~7;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(scales), 0, full_end * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rz =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(zsrc), 0, full_end * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_all =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(scales), 0, total * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rz_all =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(zsrc), 0, total * 2, 0x00020000);

    // unit loads: lane -> (row 8 h + lane / 8, permuted piece); rows past N clamped
    int vw[T][2];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = 8 * h + (lane >> 3);
            const int c = (lane & 7) ^ ((r >> 1) & 7);
            const int n = min((tile0 + t) * 16 + r, N - 1);
            vw[t][h] = n * (K >> 1) + 16 * c;
        }
    int rslot[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) rslot[e] = 8 * n16 + ((4 * e + q) ^ ((n16 >> 1) & 7));
    // activation fragment offset of this lane; rows >= M point past the buffer (zeros)
    const int xoff = n16 < M ? (n16 * K + 32 * q) * 2 : 0x40000000;
    auto load_x = [&](XStage& xs, int kp, bool live) {
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                xs.x[e][j] = __builtin_amdgcn_raw_buffer_load_b128(live ? rx : none, xoff + e * 256 + 16 * j,
                                                                   kp * 512, 0);
    };

    // 1. (scale, zero) staging loads, the first pair's activations, then the ring: pair
    //    kp0 + p of tile t into slot p * T + t
    const int sz_first = row_begin * G;
    const int sz_al = sz_first & ~7;
    const int sz_pieces = ((row_end - row_begin) * G + (sz_first - sz_al) + 7) >> 3;
    //    Waves without staging pieces load through `none` (no memory access): a branch
    //    around the loads would make the compiler wait for them at the join.
    u32x4 sv[kSzPieces], zv[kSzPieces];
#pragma unroll
    for (int j = 0; j < kSzPieces; ++j) {
        const int off = (sz_al + 8 * min(tid + NTH * j, sz_pieces - 1)) * 2;
        const bool own = (wave + W * j) * 64 < sz_pieces;            // wave-uniform
        sv[j] = __builtin_amdgcn_raw_buffer_load_b128(own ? rs : none, off, 0, 0);
        zv[j] = __builtin_amdgcn_raw_buffer_load_b128(own ? rz : none, off, 0, 0);
    }
    const int tail = min(full_end + (tid & 7), total - 1);
    const uint16_t s_tail = __builtin_amdgcn_raw_buffer_load_b16(rs_all, tail * 2, 0, 0);
    const uint16_t z_tail = __builtin_amdgcn_raw_buffer_load_b16(rz_all, tail * 2, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    XStage xr;
    load_x(xr, kp0, np > 0);
    static_for<0, PK>([&](auto pc) {
        constexpr int p = decltype(pc)::value;
        static_for<0, T>([&](auto tc) {
            constexpr int t = decltype(tc)::value;
            ring_fill<p * T + t>(p < np && t < ntiles ? rw : none, wave, vw[t], kp0 + p);
        });
    });
    __builtin_amdgcn_sched_barrier(0);

    // 2. (scale | zero << 16) words; NULL zeros become 8.0 (0x4800).  Branch-free: threads
    //    without a piece (or tail half) write the spare words at `spare` (a store under a
    //    branch would pull its load into the branch, behind a wait for every load).
    const int spare = 8 * sz_pieces;                 // 12 spare words after the staged ones
#pragma unroll
    for (int j = 0; j < kSzPieces; ++j) {
        const int p = tid + NTH * j;
        const u32x4 sw = sv[j];
        const u32x4 zw = has_zeros ? zv[j] : u32x4{0x48004800u, 0x48004800u, 0x48004800u, 0x48004800u};
        const bool ok = p < sz_pieces && sz_al + 8 * p + 8 <= total;
        u32x4* dst = reinterpret_cast<u32x4*>(szs + (ok ? 8 * p : spare));
        dst[0] = u32x4{perm(zw.x, sw.x, 0x05040100u), perm(zw.x, sw.x, 0x07060302u),
                       perm(zw.y, sw.y, 0x05040100u), perm(zw.y, sw.y, 0x07060302u)};
        dst[1] = u32x4{perm(zw.z, sw.z, 0x05040100u), perm(zw.z, sw.z, 0x07060302u),
                       perm(zw.w, sw.w, 0x05040100u), perm(zw.w, sw.w, 0x07060302u)};
    }
    {
        const int h = full_end + tid;
        const bool ok = tid < 8 && h < total && h >= sz_al && h < sz_al + 8 * sz_pieces;
        szs[ok ? h - sz_al : spare + 8] =
            (uint32_t)s_tail | ((uint32_t)(has_zeros ? z_tail : (uint16_t)0x4800) << 16);
    }
    //    Barrier on the staging stores only: __syncthreads() would also wait for the
    //    ring's loads (they write LDS), which each wave reads only itself.
    __builtin_amdgcn_s_waitcnt(0xC07F);               // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();

    int szo[T];
#pragma unroll
    for (int t = 0; t < T; ++t) szo[t] = (sz_first - sz_al) + (t * 16 + n16) * G;
    f32x4 tile[T];
#pragma unroll
    for (int t = 0; t < T; ++t) tile[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const uint32_t ones_lo = DT == DT_F16 ? 0x00010001u : 0x3F803F80u;
    const uint32_t ones_hi = DT == DT_F16 ? 0x00100010u : 0x3F803F80u;
    const uint32_t ones[4] = {ones_lo, ones_hi, ones_lo, ones_hi};

    // One k-block pair (ring slots p * T ..): activations to pair order and their sums, the
    // next pair's activations into the freed registers, then every tile's unit; REFILL
    // issues the unit PK pairs ahead into the slot just read (unconditionally, zeros past
    // the slice, so the compiler's load counts stay exact).  Deeper activation prefetch was
    // measured slower (more registers, same waits).
    auto kpair = [&](auto pc, int kp, auto refill) {
        constexpr int p = decltype(pc)::value;
        constexpr bool REFILL = decltype(refill)::value;
        uint32_t a[2][4][4];
        f32x4 S[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x4 v = xr.x[e][j];
                if constexpr (DT == DT_F16) {
                    permute_x8(v.x, v.y, v.z, v.w, a[e][j]);
                    const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
                    a[e][j][1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, a[e][j][1]) * sixteenth);
                    a[e][j][3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, a[e][j][3]) * sixteenth);
                } else {
                    permute_x8_byte(v.x, v.y, v.z, v.w, a[e][j]);
                }
            }
            S[e] = mfma16<DT>(a[e][0], ones, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
            for (int j = 1; j < 4; ++j) S[e] = mfma16<DT>(a[e][j], ones, S[e]);
        }
        load_x(xr, kp + 1, kp + 1 < kp1);             // zeros past the slice
        int grp[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) grp[e] = ((2 * kp + e) << 7) >> gshift;
        static_for<0, T>([&](auto tc) {
            constexpr int t = decltype(tc)::value;
            constexpr int d = p * T + t;
            if (t < ntiles) {                         // wave-uniform
                const u32x4* slot = ring_slot<d>(wave);
                u32x4 wb[2];
                wb[0] = slot[rslot[0]];
                wb[1] = slot[rslot[1]];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    uint32_t bq[4][4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if constexpr (DT == DT_F16)
                            unpack_mask_f16(wb[e][j], bq[j]);
                        else
                            unpack_byte<0x43>(wb[e][j], bq[j]);
                    }
                    f32x4 acc = mfma16<DT>(a[e][0], bq[0], f32x4{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
                    for (int j = 1; j < 4; ++j) acc = mfma16<DT>(a[e][j], bq[j], acc);
                    const uint32_t sz = szs[szo[t] + grp[e]];
                    const float s = h2f((uint16_t)(sz & 0xFFFFu));
                    const float z = h2f((uint16_t)(sz >> 16));
                    const float sp = DT == DT_F16 ? s * 16777216.0f : s;
                    const float c = DT == DT_F16 ? z : 128.0f + z;
#pragma unroll
                    for (int j = 0; j < 4; ++j) tile[t][j] = fmaf(sp, fmaf(-c, S[e][j], acc[j]), tile[t][j]);
                }
            }
            if constexpr (REFILL)
                ring_fill<d>(kp + PK < kp1 && t < ntiles ? rw : none, wave, vw[t], kp + PK);
        });
    };

    // 3. Rounds of PK pairs; the main loop runs while another round follows, the last
    //    round computes what is in flight without refills.
    int i = 0;
    for (; i + PK < np; i += PK)
        static_for<0, PK>([&](auto pc) { kpair(pc, kp0 + i + decltype(pc)::value, std::true_type{}); });
    static_for<0, PK>([&](auto pc) {
        if (i + decltype(pc)::value < np) kpair(pc, kp0 + i + decltype(pc)::value, std::false_type{});
    });

    // 4. Sum the waves' partial tiles through the ring (all loads landed first: the main
    //    loop's last refills past the slice are zero loads still on their way); wave t
    //    reduces tile t; lane (n, q) element j is row 4 q + j.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    static_for<0, T>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        ring_slot<t / 2>(wave)[64 * (t % 2) + lane] = __builtin_bit_cast(u32x4, tile[t]);
    });
    __syncthreads();
    static_for<0, T>([&](auto tc) {
        constexpr int t = decltype(tc)::value;
        if (wave == t && t < ntiles) {
            f32x4 v = __builtin_bit_cast(f32x4, ring_slot<t / 2>(0)[64 * (t % 2) + lane]);
#pragma unroll
            for (int w = 1; w < W; ++w) {
                const f32x4 u = __builtin_bit_cast(f32x4, ring_slot<t / 2>(w)[64 * (t % 2) + lane]);
                v[0] += u[0]; v[1] += u[1]; v[2] += u[2]; v[3] += u[3];
            }
            const int n = (tile0 + t) * 16 + n16;
            if (n < N) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int m = 4 * q + j;
                    if (m < M) Y[(size_t)m * N + n] = f2out<DT>(v[j]);
                }
            }
        }
    });
}

template <int DT, int T, int PK>
__global__ __launch_bounds__(64 * kWaves) void decode_ring_kernel(
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int has_zeros,
    uint16_t* __restrict__ Y, int M, int N, int K, int G, int gshift, int NT, int nblk, int KSP) {
    ring_block<DT, T, PK>(X, qw, scales, zeros, has_zeros, Y, M, N, K, G, gshift, NT, nblk, KSP, blockIdx.x);
}

// Grouped launch of independent layers on the ring kernel: one grid over the layers' blocks
// (block b works for the layer whose block range holds b), so the layers' latency chains
// (the weight and activation round trips of a block) overlap instead of running one launch
// after another.  A tile's arithmetic does not depend on the block that holds it, so each
// output is bit-identical to the layer's own launch on the ring kernel.
constexpr int kRingGroupMax = 16;

struct RingGroupItem {
    const uint16_t* X;
    const uint32_t* qw;
    const uint16_t* scales;
    const uint16_t* zeros;
    uint16_t* Y;
    int has_zeros, M, N, K, G, gshift, NT, nblk, ksp;
    int block_begin;       // first grid block of this layer
};

struct RingGroupArgs {
    RingGroupItem it[kRingGroupMax];
    int count;
};

template <int DT, int T, int PK>
__global__ __launch_bounds__(64 * kWaves) void decode_ring_group_kernel(const RingGroupArgs ga) {
    const int b = blockIdx.x;
    int i = 0;
#pragma unroll
    for (int j = 1; j < kRingGroupMax; ++j)
        if (j < ga.count && b >= ga.it[j].block_begin) i = j;
    const RingGroupItem& t = ga.it[i];
    ring_block<DT, T, PK>(t.X, t.qw, t.scales, t.zeros, t.has_zeros, t.Y, t.M, t.N, t.K, t.G, t.gshift, t.NT,
                          t.nblk, t.ksp, b - t.block_begin);
}

struct DecCfg {
    int t = 0, p = 0, ksp = 0, nblk = 0;
    int sk = 0, spare = 0, szs = 0, wt = 0, lds = 0;
};

DecCfg pick_decode_staged(const LinearArgs& a) {
    DecCfg c;
    if (a.M < 1 || a.M > 4 || a.K % 256 != 0 || a.g % 128 != 0) return c;
    // 32-bit buffer offsets
    if ((long long)a.N * (a.K / 2) >= (1LL << 31) || (long long)a.M * a.K * 2 >= (1LL << 31)) return c;
    if ((long long)a.N * a.G * 2 >= (1LL << 31)) return c;
    const int NT = (a.N + 15) / 16;
    const int KB = a.K / 128;
    // tiles per block: the fewest that keep the grid within one block per CU (at most 4)
    int t = (NT + 255) / 256;
    if (t > 4) t = 4;
    const int ksp = (KB / 2 + kWaves - 1) / kWaves;
    const int xpitch = KB * 128 + 8;
    const long long pieces = ((long long)t * 16 * a.G + 7) / 8 + 1;
    if (pieces > (long long)kSzPieces * 64 * kWaves) return c;
    c.sk = align16(a.M * xpitch * 2);
    c.spare = align16(c.sk + KB * 16);
    c.szs = c.spare + 32;
    c.wt = align16(c.szs + (int)pieces * 32);
    long long lds = (long long)c.wt + (long long)kWaves * 2048;
    const long long red = (long long)kWaves * t * 1024;      // final reduction, from offset 0
    if (red > lds) lds = red;
    if (lds > kLdsBudget) return c;
    c.lds = (int)lds;
    c.t = t;
    // k-block pairs in flight: about twelve 16-byte loads per lane, fewer for M > 1
    // (register budget of two waves per SIMD)
    if (a.M == 1)
        c.p = t == 1 ? (ksp <= 2 ? 2 : 6) : (t == 2 ? 3 : 2);
    else
        c.p = t == 1 ? (ksp <= 2 ? 2 : 3) : (t == 4 ? 1 : 2);
    c.ksp = ksp;
    c.nblk = (NT + t - 1) / t;
    return c;
}

template <int DT, int M, int T, int P>
hipError_t run(const LinearArgs& a, const DecCfg& c, hipStream_t st) {
    hipLaunchKernelGGL((decode_kernel<DT, M, T, P, kWaves>), dim3(c.nblk), dim3(64 * kWaves), c.lds, st,
                       static_cast<const uint16_t*>(a.X), a.qw, a.scales, a.zeros, a.zeros ? 1 : 0,
                       static_cast<uint16_t*>(a.Y), a.N, a.K, a.G, a.gshift, (a.N + 15) / 16, c.nblk,
                       c.ksp, c.sk, c.spare, c.szs, c.wt);
    return hipGetLastError();
}

template <int DT, int M>
hipError_t run_m(const LinearArgs& a, const DecCfg& c, hipStream_t st) {
    if constexpr (M == 1) {
        if (c.t == 1) return c.p == 2 ? run<DT, M, 1, 2>(a, c, st) : run<DT, M, 1, 6>(a, c, st);
        if (c.t == 2) return run<DT, M, 2, 3>(a, c, st);
        if (c.t == 3) return run<DT, M, 3, 2>(a, c, st);
        return run<DT, M, 4, 2>(a, c, st);
    } else {
        if (c.t == 1) return c.p == 2 ? run<DT, M, 1, 2>(a, c, st) : run<DT, M, 1, 3>(a, c, st);
        if (c.t == 2) return run<DT, M, 2, 2>(a, c, st);
        if (c.t == 3) return run<DT, M, 3, 2>(a, c, st);
        return run<DT, M, 4, 1>(a, c, st);
    }
}

template <int DT>
hipError_t run_dt(const LinearArgs& a, const DecCfg& c, hipStream_t st) {
    switch (a.M) {
        case 1: return run_m<DT, 1>(a, c, st);
        case 2: return run_m<DT, 2>(a, c, st);
        case 3: return run_m<DT, 3>(a, c, st);
        case 4: return run_m<DT, 4>(a, c, st);
    }
    return hipErrorInvalidValue;
}

// The ring kernel: T tiles per block, about one block per CU (T = NT / 256, at most 8, fewer
// when the block's (scale, zero) words would not fit); PK pairs in flight per wave, two up to
// four tiles and one beyond (PK * T <= 8 slots).  Measured against holding the weight loads
// in registers (16 rows; 4096 -> 4096, 4096 -> 11008, 11008 -> 4096, 8192 -> 28672,
// 28672 -> 8192): 7.0 / 10.1 / 13.9 / 26.9 / 37.3 us against 7.3 / 11.1 / 14.1 / 34.2 /
// 38.1 us.  Deeper rings for few tiles (four pairs) were slower.
struct RingCfg {
    int t = 0, pk = 0, ksp = 0, nblk = 0, lds = 0;
};

constexpr int kLdsPerCu = 160 * 1024;

constexpr int ring_pk(int t) { return t <= 4 ? 2 : 1; }
constexpr long long ring_bytes(int t) { return (long long)t * ring_pk(t) * kWaves * kRingUnit * 16; }

bool ring_shape_ok(const LinearArgs& a) {
    if (a.M < 1 || a.M > 16 || a.K % 256 != 0 || a.g % 128 != 0) return false;
    if ((long long)a.N * (a.K / 2) >= (1LL << 31) || (long long)a.M * a.K * 2 >= (1LL << 30)) return false;
    return (long long)a.N * a.G * 2 < (1LL << 31);
}

// The configuration with t tiles per block, or t == 0 when its staging or LDS does not fit.
RingCfg ring_cfg(const LinearArgs& a, int t) {
    RingCfg c;
    const long long pieces = ((long long)t * 16 * a.G + 7) / 8 + 1;
    if (pieces > (long long)kSzPieces * 64 * kWaves) return c;
    const long long dyn = align16((int)pieces * 32 + 48);              // + spare words
    if (dyn + ring_bytes(t) > kLdsPerCu) return c;
    const int NT = (a.N + 15) / 16;
    c.t = t;
    c.pk = ring_pk(t);
    c.ksp = (a.K / 256 + kWaves - 1) / kWaves;
    c.nblk = (NT + t - 1) / t;
    c.lds = (int)dyn;
    return c;
}

RingCfg pick_ring(const LinearArgs& a) {
    if (!ring_shape_ok(a)) return RingCfg{};
    const int NT = (a.N + 15) / 16;
    for (int t = std::min(kRingSlots, (NT + 255) / 256); t >= 1; --t) {
        const RingCfg c = ring_cfg(a, t);
        if (c.t > 0) return c;
    }
    return RingCfg{};
}

template <int DT, int T, int PK>
hipError_t run_ring3(const LinearArgs& a, const RingCfg& c, hipStream_t st) {
    hipLaunchKernelGGL((decode_ring_kernel<DT, T, PK>), dim3(c.nblk), dim3(64 * kWaves), c.lds, st,
                       static_cast<const uint16_t*>(a.X), a.qw, a.scales, a.zeros, a.zeros ? 1 : 0,
                       static_cast<uint16_t*>(a.Y), a.M, a.N, a.K, a.G, a.gshift, (a.N + 15) / 16, c.nblk,
                       c.ksp);
    return hipGetLastError();
}

template <int DT>
hipError_t run_ring(const LinearArgs& a, const RingCfg& c, hipStream_t st) {
    switch (c.t) {
        case 1: return run_ring3<DT, 1, 2>(a, c, st);
        case 2: return run_ring3<DT, 2, 2>(a, c, st);
        case 3: return run_ring3<DT, 3, 2>(a, c, st);
        case 4: return run_ring3<DT, 4, 2>(a, c, st);
        case 5: return run_ring3<DT, 5, 1>(a, c, st);
        case 6: return run_ring3<DT, 6, 1>(a, c, st);
        case 7: return run_ring3<DT, 7, 1>(a, c, st);
        case 8: return run_ring3<DT, 8, 1>(a, c, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

// M <= 4 prefers the activation-staging kernel; when the activations do not fit its LDS
// (long K), or M > 4, the ring kernel.
bool decode_supports(const LinearArgs& a) {
    return (a.M <= 4 && pick_decode_staged(a).t > 0) || pick_ring(a).t > 0;
}

hipError_t launch_decode(const LinearArgs& a, hipStream_t st) {
    if (a.M <= 4) {
        const DecCfg c = pick_decode_staged(a);
        if (c.t > 0) return a.dtype == DT_F16 ? run_dt<DT_F16>(a, c, st) : run_dt<DT_BF16>(a, c, st);
    }
    const RingCfg rc = pick_ring(a);
    if (rc.t == 0) return hipErrorInvalidValue;
    return a.dtype == DT_F16 ? run_ring<DT_F16>(a, rc, st) : run_ring<DT_BF16>(a, rc, st);
}

namespace {
// A layer joins a grouped launch with one tile per block: up to 8 activation rows and rows
// and columns of at most 12288, where the blocks are small (32 KB of ring, two blocks per
// CU), the layers' blocks overlap, and the activations re-read by the extra blocks (2 M
// bytes per column against 8 bytes of weights per tile) stay within L2's reach.  Measured on
// the 7B-like step (three layers, one batch call against three calls): M = 4: 23.4 -> 20.3
// us, M = 8: 25.7 -> 23.1 us; larger layers (8192 -> 28672, 28672 -> 8192) and M = 16 were
// slower grouped (M = 8, 70B-like step: 64.5 -> 87.6 us with one tile per block).
RingCfg ring_group_cfg(const LinearArgs& a) {
    if (a.M > 8 || a.N > 12288 || a.K > 12288 || pick_ring(a).t == 0) return RingCfg{};
    return ring_cfg(a, 1);
}
}  // namespace

bool ring_group_supports(const LinearArgs& a) { return ring_group_cfg(a).t > 0; }

hipError_t launch_ring_group(const LinearArgs* items, int count, hipStream_t st) {
    if (count < 1 || count > kRingGroupMax) return hipErrorInvalidValue;
    // every layer of the group runs one tile per block (ring_group_cfg), each within the LDS
    int lds = 0;
    RingCfg cfg[kRingGroupMax];
    for (int i = 0; i < count; ++i) {
        if (items[i].dtype != items[0].dtype) return hipErrorInvalidValue;
        cfg[i] = ring_group_cfg(items[i]);
        if (cfg[i].t != 1) return hipErrorInvalidValue;
        lds = std::max(lds, cfg[i].lds);
    }
    // blocks of the layers with the longest rows (the longest-lived blocks) are dispatched first
    int order[kRingGroupMax];
    for (int i = 0; i < count; ++i) order[i] = i;
    std::stable_sort(order, order + count, [&](int x, int y) { return items[x].K > items[y].K; });
    RingGroupArgs ga{};
    ga.count = count;
    long long blocks = 0;
    for (int oi = 0; oi < count; ++oi) {
        const LinearArgs& a = items[order[oi]];
        const RingCfg& c = cfg[order[oi]];
        RingGroupItem& t = ga.it[oi];
        t.X = static_cast<const uint16_t*>(a.X);
        t.qw = a.qw;
        t.scales = a.scales;
        t.zeros = a.zeros;
        t.Y = static_cast<uint16_t*>(a.Y);
        t.has_zeros = a.zeros ? 1 : 0;
        t.M = a.M;
        t.N = a.N;
        t.K = a.K;
        t.G = a.G;
        t.gshift = a.gshift;
        t.NT = (a.N + 15) / 16;
        t.nblk = c.nblk;
        t.ksp = c.ksp;
        t.block_begin = (int)blocks;
        blocks += c.nblk;
    }
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (items[0].dtype == DT_F16)
        hipLaunchKernelGGL((decode_ring_group_kernel<DT_F16, 1, ring_pk(1)>), dim3((unsigned)blocks),
                           dim3(64 * kWaves), lds, st, ga);
    else
        hipLaunchKernelGGL((decode_ring_group_kernel<DT_BF16, 1, ring_pk(1)>), dim3((unsigned)blocks),
                           dim3(64 * kWaves), lds, st, ga);
    return hipGetLastError();
}

}  // namespace w4a16
