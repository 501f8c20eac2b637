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
// h / (Hq / Hkv), for one sequence or a batch of sequences with their own lengths (caches
// [B, Hkv, Tmax, D]), in two launches (split over tokens, then a merge):
//   split kernel, block (split, group of query heads, sequence), 256 threads: a cached row is
//   read by a few consecutive lanes with one 16-byte load each, so a wave load covers 8-32
//   whole rows (1-2 KB contiguous); scores (v_dot2 on exact 16-bit codes for fp16 queries)
//   are reduced across those lanes with DPP, and every lane keeps an online softmax (running
//   max, sum, output segment) over the rows it reads; the slots and the waves are combined at
//   the end into the split's (max, sum, unnormalized output);
//   merge kernel: rescales the splits to the common max and normalizes.
// Dequantization happens in registers only; the cache is read once per group of query heads.
#include "common.h"
#include "launch.h"

namespace w4a16 {

namespace {

constexpr int kKvThreads = 256;
// Token splits per head: about kKvBlocks split blocks over all heads, at least kKvMinRows rows
// each (so at most kKvBlocks splits of one head).
#ifndef W4A16_KV_MIN_ROWS
#define W4A16_KV_MIN_ROWS 256
#endif
#ifndef W4A16_KV_LOADS
#define W4A16_KV_LOADS 4
#endif
constexpr int kKvBlocks = 2048;
constexpr int kKvMinRows = W4A16_KV_MIN_ROWS;

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

// Geometry of the split kernel: a cached row of RB bytes is read by LPR consecutive lanes with
// one 16-byte load each (EPL codes per lane), so one wave load covers RPW whole rows, and a
// wave takes U such loads of K (and of V) per iteration.
template <int BITS, int D>
struct KvGeom {
    static constexpr int RB = BITS == 8 ? D : D / 2;
    static constexpr int LPR = RB / 16;
    static constexpr int RPW = 64 / LPR;
    static constexpr int EPL = D / LPR;
    static constexpr int U = W4A16_KV_LOADS;
    static constexpr int ROWS_IT = RPW * U;
};

// Sum over the LPR (2, 4 or 8) consecutive lanes of a row group; every lane of the group gets
// the same bits (each step adds the same two operands in both lanes of a pair).
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
    v += dpp_mov<0xB1>(v);                          // quad_perm [1,0,3,2]
    if constexpr (LPR >= 4) v += dpp_mov<0x4E>(v);  // quad_perm [2,3,0,1]
    if constexpr (LPR >= 8) v += dpp_mov<0x141>(v); // row_half_mirror
    return v;
}

// The 16 (KV8) or 32 (KV4) codes of a 16-byte load, lowest address first, as floats, one
// byte-to-float conversion each.  KV8 codes come out offset by +128 (the sign bit flipped, so
// every byte is unsigned); the caller removes the offset with one term per row.
template <int BITS>
__device__ __forceinline__ void codes16(const u32x4& w, float* c) {
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if constexpr (BITS == 8) {
            const uint32_t u = ww[k] ^ 0x80808080u;
#pragma unroll
            for (int i = 0; i < 4; ++i) c[4 * k + i] = (float)((u >> (8 * i)) & 0xFFu);
        } else {
            uint32_t lo = ww[k] & 0x0F0F0F0Fu;                // codes 0, 2, 4, 6
            uint32_t hi = (ww[k] >> 4) & 0x0F0F0F0Fu;         // codes 1, 3, 5, 7
            // opaque to the optimizer, so each byte below stays one byte-to-float conversion
            // instead of being refolded into a bit-field extract plus a conversion
            asm volatile("" : "+v"(lo), "+v"(hi));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                c[8 * k + 2 * i] = (float)((lo >> (8 * i)) & 0xFFu);
                c[8 * k + 2 * i + 1] = (float)((hi >> (8 * i)) & 0xFFu);
            }
        }
    }
}

// One block = one token split x GQ query heads that share a kv head.  Lane (slot, seg) reads
// segment seg of row slot of every wave load and keeps, per query head, its own running max m,
// sum l and unnormalized output segment (online softmax over the rows of its slot); scores are
// in the base-2 domain (q is prescaled by log2(e) / sqrt(D)).  At the end the slots and the
// four waves are combined and the block's (m, l, o[D]) goes to the workspace.
template <int DT, int BITS, int D, int GQ>
__global__ __launch_bounds__(kKvThreads) void kv_attn_split_kernel(
    const uint16_t* __restrict__ q, int Hq, int Hkv, int T, const int* __restrict__ lens, int Tmax, int chunk,
    const void* __restrict__ kc, const uint16_t* __restrict__ ks, const uint16_t* __restrict__ kz,
    const void* __restrict__ vc, const uint16_t* __restrict__ vs, const uint16_t* __restrict__ vz,
    float* __restrict__ part) {
    using G = KvGeom<BITS, D>;
    constexpr int RB = G::RB, LPR = G::LPR, RPW = G::RPW, EPL = G::EPL, U = G::U;
    constexpr int NW = kKvThreads / 64;
    __shared__ float pacc[GQ][NW][D];
    __shared__ float pm[GQ][NW], pl[GQ][NW];
    const int split = blockIdx.x;
    const int nsplit = gridDim.x;
    const int h0 = blockIdx.y * GQ;
    const int kvh = h0 / (Hq / Hkv);
    // sequence b of the batch: its length (clamped into [1, Tmax]) and its heads
    const int b = blockIdx.z;
    if (lens) T = min(max(lens[b], 1), Tmax);
    const long long hq0 = (long long)b * Hq + h0;       // first query head of the block, batch-wide
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int seg = lane % LPR, slot = lane / LPR;
    const int t0 = split * chunk;
    const int t1 = min(T, t0 + chunk);
    const long long rowbase = ((long long)b * Hkv + kvh) * Tmax;
    const float NEG = -__builtin_inff();

    // uniform per-head bases and 32-bit per-lane offsets (Tmax * RB < 2^32)
    const unsigned char* kb = static_cast<const unsigned char*>(kc) + rowbase * RB;
    const unsigned char* vb = static_cast<const unsigned char*>(vc) + rowbase * RB;
    const uint16_t* ksb = ks + rowbase;
    const uint16_t* vsb = vs + rowbase;
    const uint16_t* kzb = BITS == 4 ? kz + rowbase : nullptr;
    const uint16_t* vzb = BITS == 4 ? vz + rowbase : nullptr;
    constexpr int STRIDE = NW * G::ROWS_IT;

    // The loads of one wave iteration (rows base + u RPW + slot); rows past the split are
    // clamped to its last row (always in the cache) and masked out of the softmax.
    struct Raw {
        u32x4 kw[U], vw[U];
        uint16_t ks[U], vs[U], kz[U], vz[U];
    };
    auto issue = [&](int base, Raw& R) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = base + u * RPW + slot;
            const uint32_t row = (uint32_t)(r < t1 ? r : t1 - 1);
            const uint32_t off = row * (uint32_t)RB + 16u * (uint32_t)seg;
            R.kw[u] = *reinterpret_cast<const u32x4*>(kb + off);
            R.vw[u] = *reinterpret_cast<const u32x4*>(vb + off);
            R.ks[u] = ksb[row];
            R.vs[u] = vsb[row];
            if constexpr (BITS == 4) {
                R.kz[u] = kzb[row];
                R.vz[u] = vzb[row];
            }
        }
    };

    // the query's loads, then the first iteration's, are issued before either is waited on
    const int base0 = t0 + wave * G::ROWS_IT;
    u32x4 qraw[GQ][EPL / 8];
#pragma unroll
    for (int g = 0; g < GQ; ++g)
#pragma unroll
        for (int p = 0; p < EPL / 8; ++p)
            qraw[g][p] = *reinterpret_cast<const u32x4*>(q + (hq0 + g) * D + seg * EPL + 8 * p);
    Raw A;
    issue(base0, A);      // a wave with no rows reads the split's last row and masks it
    __builtin_amdgcn_sched_barrier(0);

    // this lane's segment of each query head, prescaled; its segment sum (code offset term)
    // fp16 queries score with v_dot2 on exact 16-bit codes (KV8: 1024 + (c + 128) from one
    // byte permute per pair; KV4: subnormal codes u 2^-24, half of them x16, from masks), with
    // q kept as loaded (pairs in the codes' order) and scaled after the dot product; bf16
    // queries take q prescaled in fp32 and one conversion and multiply-add per code.
    constexpr bool DOT = DT == DT_F16;
    const float qscale = 1.4426950408889634f / sqrtf((float)D);
    float qv[GQ][DOT ? 1 : EPL], qseg[GQ];
    uint32_t qp[GQ][DOT ? EPL / 2 : 1];
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
        qseg[g] = 0.0f;
#pragma unroll
        for (int p = 0; p < EPL / 8; ++p) {
            const uint32_t ww[4] = {qraw[g][p].x, qraw[g][p].y, qraw[g][p].z, qraw[g][p].w};
            if constexpr (DOT) {
                if constexpr (BITS == 8) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) qp[g][4 * p + i] = ww[i];
                } else {
                    permute_x8(ww[0], ww[1], ww[2], ww[3], &qp[g][4 * p]);
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) qseg[g] += h2f((ww[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    qv[g][8 * p + i] = in2f<DT>((ww[i >> 1] >> (16 * (i & 1))) & 0xFFFFu) * qscale;
                    qseg[g] += qv[g][8 * p + i];
                }
            }
        }
    }
    float m[GQ], l[GQ], acc[GQ][EPL], zoff[GQ];
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
        m[g] = NEG;
        l[g] = 0.0f;
        zoff[g] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = 0.0f;
    }

    // online-softmax update with the rows of one iteration
    auto consume = [&](int base, const Raw& R, auto first) {
        float sc[GQ][U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = base + u * RPW + slot < t1;
            if constexpr (DOT) {
                const float kq = h2f(R.ks[u]) * qscale;
                const uint32_t ww[4] = {R.kw[u].x, R.kw[u].y, R.kw[u].z, R.kw[u].w};
                if constexpr (BITS == 8) {
                    uint32_t h16[8];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint32_t b = ww[k] ^ 0x80808080u;            // c + 128 per byte
                        h16[2 * k] = perm(0x64646464u, b, 0x04010400u);    // (1024 + b0, 1024 + b1)
                        h16[2 * k + 1] = perm(0x64646464u, b, 0x04030402u);
                    }
#pragma unroll
                    for (int g = 0; g < GQ; ++g) {
                        float d = 0.0f;
#pragma unroll
                        for (int i = 0; i < 8; ++i) d = dot2<DT_F16>(qp[g][i], h16[i], d);
                        d = fmaf(-1152.0f, qseg[g], d);
                        d = group_sum<LPR>(d);
                        sc[g][u] = ok ? d * kq : NEG;
                    }
                } else {
                    uint32_t cd[4][4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) unpack_mask_f16(ww[k], cd[k]);
#pragma unroll
                    for (int g = 0; g < GQ; ++g) {
                        float pa = 0.0f, pb = 0.0f;
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            pa = dot2<DT_F16>(qp[g][4 * k + 0], cd[k][0], pa);
                            pb = dot2<DT_F16>(qp[g][4 * k + 1], cd[k][1], pb);
                            pa = dot2<DT_F16>(qp[g][4 * k + 2], cd[k][2], pa);
                            pb = dot2<DT_F16>(qp[g][4 * k + 3], cd[k][3], pb);
                        }
                        float d = fmaf(pb, 0.0625f, pa) * 16777216.0f;     // sum q u
                        d = fmaf(-h2f(R.kz[u]), qseg[g], d);
                        d = group_sum<LPR>(d);
                        sc[g][u] = ok ? d * kq : NEG;
                    }
                }
            } else {
                const float ksc = h2f(R.ks[u]);
                float c[EPL];
                codes16<BITS>(R.kw[u], c);
#pragma unroll
                for (int g = 0; g < GQ; ++g) {
                    float d = 0.0f;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) d = fmaf(qv[g][e], c[e], d);
                    d = fmaf(BITS == 4 ? -h2f(R.kz[u]) : -128.0f, qseg[g], d);
                    d = group_sum<LPR>(d);
                    sc[g][u] = ok ? d * ksc : NEG;
                }
            }
        }
        float pv[GQ][U];
#pragma unroll
        for (int g = 0; g < GQ; ++g) {
            float mt = sc[g][0];
#pragma unroll
            for (int u = 1; u < U; ++u) mt = fmaxf(mt, sc[g][u]);
            const float mn = fmaxf(m[g], mt);
            const bool any = mn != NEG;
            const float corr = any ? exp2f(m[g] - mn) : 1.0f;
            float ps = 0.0f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float p = any ? exp2f(sc[g][u] - mn) : 0.0f;
                ps += p;
                pv[g][u] = p * h2f(R.vs[u]);
            }
            m[g] = mn;
            if constexpr (decltype(first)::value) {     // nothing accumulated yet
                l[g] = ps;
            } else {
                l[g] = fmaf(l[g], corr, ps);
                zoff[g] *= corr;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[g][e] *= corr;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float c[EPL];
            codes16<BITS>(R.vw[u], c);
#pragma unroll
            for (int g = 0; g < GQ; ++g) {
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(pv[g][u], c[e], acc[g][e]);
                zoff[g] = fmaf(pv[g][u], BITS == 4 ? h2f(R.vz[u]) : 128.0f, zoff[g]);
            }
        }
    };

    // (a consume whose rows are all masked changes nothing)
    consume(base0, A, std::true_type{});
    for (int base = base0 + STRIDE; base < t1; base += STRIDE) {
        issue(base, A);
        __builtin_amdgcn_sched_barrier(0);
        consume(base, A, std::false_type{});
    }

    // combine the slots of the wave (lanes with the same segment), then the waves
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
        float M = m[g];
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
        const float f = m[g] == NEG ? 0.0f : exp2f(m[g] - M);
        float lw = l[g] * f;
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) lw += __shfl_xor(lw, off, 64);
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            float a = (acc[g][e] - zoff[g]) * f;
#pragma unroll
            for (int off = LPR; off < 64; off <<= 1) a += __shfl_xor(a, off, 64);
            acc[g][e] = a;
        }
        if (slot == 0) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) pacc[g][wave][seg * EPL + e] = acc[g][e];
            if (seg == 0) {
                pm[g][wave] = M;
                pl[g][wave] = lw;
            }
        }
    }
    __syncthreads();
    for (int idx = tid; idx < GQ * D; idx += kKvThreads) {
        const int g = idx / D, d = idx % D;
        float M = pm[g][0];
#pragma unroll
        for (int w = 1; w < NW; ++w) M = fmaxf(M, pm[g][w]);
        float o = 0.0f, lt = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float f = pm[g][w] == NEG ? 0.0f : exp2f(pm[g][w] - M);
            o = fmaf(pacc[g][w][d], f, o);
            lt = fmaf(pl[g][w], f, lt);
        }
        float* out = part + ((hq0 + g) * nsplit + split) * (D + 2);
        out[2 + d] = o;
        if (d == 0) {
            out[0] = M;
            out[1] = lt;
        }
    }
}

// One block per query head.  Thread (phase, d) folds output dimension d of splits phase,
// phase + PH, ... into a running (max, sum, output), eight splits per step with all their loads
// independent (a head with up to 8 PH splits takes one memory round trip); the PH phases are
// then combined through LDS.
template <int DT, int D>
__global__ __launch_bounds__(256) void kv_attn_merge_kernel(const float* __restrict__ part, int nsplit,
                                                            uint16_t* __restrict__ out) {
    constexpr int PH = 256 / D;
    constexpr int S = 8;
    __shared__ float sm[PH][D], sl[PH][D], so[PH][D];
    const long long h = blockIdx.x;                     // batch-wide query head
    const int tid = threadIdx.x;
    const int d = tid % D, ph = tid / D;
    const float NEG = -__builtin_inff();
    const float* p = part + (long long)h * nsplit * (D + 2);
    float M = NEG, L = 0.0f, O = 0.0f;
    for (int j0 = ph; j0 < nsplit; j0 += S * PH) {
        float mj[S], lj[S], oj[S];
#pragma unroll
        for (int i = 0; i < S; ++i) {
            const int j = j0 + i * PH;
            const long long at = (long long)(j < nsplit ? j : j0) * (D + 2);
            mj[i] = p[at];
            lj[i] = p[at + 1];
            oj[i] = p[at + 2 + d];
            if (j >= nsplit) mj[i] = NEG;
        }
        float mn = M;
#pragma unroll
        for (int i = 0; i < S; ++i) mn = fmaxf(mn, mj[i]);
        if (mn == NEG) continue;
        const float c = exp2f(M - mn);
        L *= c;
        O *= c;
#pragma unroll
        for (int i = 0; i < S; ++i) {
            const float w = mj[i] == NEG ? 0.0f : exp2f(mj[i] - mn);
            L = fmaf(lj[i], w, L);
            O = fmaf(oj[i], w, O);
        }
        M = mn;
    }
    sm[ph][d] = M;
    sl[ph][d] = L;
    so[ph][d] = O;
    __syncthreads();
    if (tid < D) {
        float mx = sm[0][tid];
#pragma unroll
        for (int k = 1; k < PH; ++k) mx = fmaxf(mx, sm[k][tid]);
        float lt = 0.0f, ot = 0.0f;
#pragma unroll
        for (int k = 0; k < PH; ++k) {
            const float w = sm[k][tid] == NEG ? 0.0f : exp2f(sm[k][tid] - mx);
            lt = fmaf(sl[k][tid], w, lt);
            ot = fmaf(so[k][tid], w, ot);
        }
        out[(long long)h * D + tid] = f2out<DT>(ot / lt);
    }
}

int kv_splits(int Hq, int T) {
    int ns = (kKvBlocks + Hq - 1) / Hq;
    ns = min(ns, (T + kKvMinRows - 1) / kKvMinRows);
    return max(ns, 1);
}

// query heads per block: those of one kv head, up to 4 (KV8) or 2 (KV4) to bound registers
template <int BITS>
int kv_group(int Hq, int Hkv) {
    const int grp = Hq / Hkv;
    if (BITS == 8 && grp % 4 == 0) return 4;
    return grp % 2 == 0 ? 2 : 1;
}

// B sequences; `lens` (device, B entries) gives each sequence's length, or NULL: every
// sequence has T tokens.  Splits are sized on the longest span (T, or Tmax with lens).
template <int DT, int BITS, int D>
hipError_t kv_attn(const void* q, int B, int Hq, int Hkv, int T, const int* lens, int Tmax, const void* kc,
                   const uint16_t* ks, const uint16_t* kz, const void* vc, const uint16_t* vs, const uint16_t* vz,
                   float* work, void* out, hipStream_t st) {
    const int span = lens ? Tmax : T;
    const int ns = kv_splits(B * Hq, span);
    const int chunk = (span + ns - 1) / ns;
    const int gq = kv_group<BITS>(Hq, Hkv);
    const auto qp = static_cast<const uint16_t*>(q);
    if (gq == 4)
        hipLaunchKernelGGL((kv_attn_split_kernel<DT, BITS, D, (BITS == 8 ? 4 : 1)>), dim3(ns, Hq / 4, B),
                           dim3(kKvThreads), 0, st, qp, Hq, Hkv, T, lens, Tmax, chunk, kc, ks, kz, vc, vs, vz, work);
    else if (gq == 2)
        hipLaunchKernelGGL((kv_attn_split_kernel<DT, BITS, D, 2>), dim3(ns, Hq / 2, B), dim3(kKvThreads), 0, st,
                           qp, Hq, Hkv, T, lens, Tmax, chunk, kc, ks, kz, vc, vs, vz, work);
    else
        hipLaunchKernelGGL((kv_attn_split_kernel<DT, BITS, D, 1>), dim3(ns, Hq, B), dim3(kKvThreads), 0, st, qp,
                           Hq, Hkv, T, lens, Tmax, chunk, kc, ks, kz, vc, vs, vz, work);
    hipLaunchKernelGGL((kv_attn_merge_kernel<DT, D>), dim3(B * Hq), dim3(256), 0, st, work, ns,
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

long long kv_attention_workspace_floats(long long B, long long Hq, long long T, long long D) {
    return B * Hq * kv_splits((int)(B * Hq), (int)T) * (D + 2);
}

hipError_t launch_kv_quantize(const void* x, int dtype, long long rows, int D, int bits, void* codes,
                              uint16_t* scales, uint16_t* zeros, hipStream_t st) {
    if (dtype == DT_F16)
        return bits == 8 ? kv_quant<DT_F16, 8>(x, rows, D, codes, scales, zeros, st)
                         : kv_quant<DT_F16, 4>(x, rows, D, codes, scales, zeros, st);
    return bits == 8 ? kv_quant<DT_BF16, 8>(x, rows, D, codes, scales, zeros, st)
                     : kv_quant<DT_BF16, 4>(x, rows, D, codes, scales, zeros, st);
}

hipError_t launch_kv_attention(const void* q, int dtype, int B, int Hq, int Hkv, int T, const int* lens, int Tmax,
                               int D, int bits, const void* kc, const uint16_t* ks, const uint16_t* kz,
                               const void* vc, const uint16_t* vs, const uint16_t* vz, float* work, void* out,
                               hipStream_t st) {
#define W4A16_KV_CASE(DTV, BV, DV)                                                                          \
    if (dtype == DTV && bits == BV && D == DV)                                                              \
        return kv_attn<DTV, BV, DV>(q, B, Hq, Hkv, T, lens, Tmax, kc, ks, kz, vc, vs, vz, work, out, st);
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
