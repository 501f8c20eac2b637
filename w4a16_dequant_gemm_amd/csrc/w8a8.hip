// W8A8 with SmoothQuant on CDNA4: smoothing factors, per-channel INT8 weights, per-token
// INT8 activations and the INT8 matrix-core product with a float epilogue.
//
// Method (page "大模型推理中 Weight-only、W8A8 和 FP8 量化有什么区别？如何选型？", section 三:
// both operands in 8 bits so the product runs on the integer matrix units, the activation
// outlier channels moved into the weights by Y = (X / s)(s W); page "推理优化中“用精度换性能“
// 的核心技术：量化", 6.2: s_j = max|X_j|^alpha / max|W_j|^(1 - alpha), alpha = 0.5; 3.3 / 3.4:
// symmetric absmax scales, per channel for weights and per token for activations; page
// "Quantization & Acceleration: 解释 W8A8 与 W4A16 的差异与取舍": per-token dynamic activation
// scales).  fp32 arithmetic in a fixed order everywhere, so codes, scales and outputs are
// reproducible bit for bit: alpha = a / 4 with powers from square roots and products; x / s
// and w * s rounded once; scale = amax / 127 (1 if 0); code = clamp(rint(v / scale), -128,
// 127); output = out(fp32(fp32(acc) * sx[m]) * sw[n]) from the exact int32 sum.
//
// GEMM.  qx [M, K] and qw [N, K] int8, K contiguous ("NT"), K % 128 == 0.  Block tile 256 x 256,
// k-step 128 bytes, 8 waves in 2 x 4 (128 x 64 each), MFMA 32x32x32 i8 (lane (r, h) holds
// bytes 16 h .. + 15 of the 32-byte k-slice; for the j-th slice of a step it reads 16-byte
// piece 4 h + j of the row, a consistent k assignment for both operands).  Both operand tiles
// go global -> LDS with buffer-load-to-LDS into XOR-swizzled double buffers (piece c of row r
// at slot c ^ (r / 2 % 8), conflict-free 32-row fragment reads); 128 KB of LDS, one block per
// CU; tiles assigned XCD-major.  Two waves per SIMD (186 registers each) keep the matrix cores
// fed while the other wave waits at a step's end; measured against 4 waves of 128 x 128 (one
// per SIMD, 6 fragment reads per 8 MFMAs here against 8 per 16): M = 4096, 4096 -> 11008:
// 288 -> 237-246 us; 11008 -> 4096: 205 -> 185-189 us (the same bits).
#include "common.h"
#include "launch.h"
#include "tile.h"

namespace w4a16 {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float pow_quarters(float v, int a) {
    const float q = sqrtf(sqrtf(v));
    float out = 1.0f;
    for (int i = 0; i < a; ++i) out = out * q;
    return out;
}

// s_j from max|X_j| (n rows of X) and max|W_:,j| (N rows of W), one thread per channel
template <int DT>
__global__ __launch_bounds__(256) void smooth_kernel(const uint16_t* __restrict__ X, int n, const float* __restrict__ W,
                                                     int N, int K, int a, float* __restrict__ s) {
    const int k = blockIdx.x * 256 + threadIdx.x;
    if (k >= K) return;
    float xm = 0.0f, wm = 0.0f;
    for (int t = 0; t < n; ++t) xm = fmaxf(xm, fabsf(in2f<DT>(X[(long long)t * K + k])));
    for (int r = 0; r < N; ++r) wm = fmaxf(wm, fabsf(W[(long long)r * K + k]));
    const float num = pow_quarters(xm, a);
    const float den = pow_quarters(wm, 4 - a);
    const float v = num / (den == 0.0f ? 1.0f : den);
    s[k] = (xm == 0.0f || wm == 0.0f) ? 1.0f : v;
}

// The same factors for K % 4 == 0 with 8-byte aligned X and 16-byte aligned W rows: a block
// owns 64 channels; thread (row group rg, column group cg) reads 4 channels of rows rg,
// rg + 64, ... with 8 rows' loads in flight (rows past the end re-read the last row: max is
// idempotent), then the 64 row groups are folded through LDS.  Same values as smooth_kernel
// (a maximum does not depend on its order).
template <int DT>
__global__ __launch_bounds__(1024) void smooth_tile_kernel(const uint16_t* __restrict__ X, int n,
                                                           const float* __restrict__ W, int N, int K, int a,
                                                           float* __restrict__ s) {
    constexpr int U = 8;
    __shared__ float red[2][64][65];
    const int tid = threadIdx.x;
    const int cg = tid & 15, rg = tid >> 4;
    const int k0 = blockIdx.x * 64 + 4 * cg;
    const int kk = k0 < K ? k0 : 0;
    float xm[4] = {0.0f, 0.0f, 0.0f, 0.0f}, wm[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int t = rg; t < n; t += 64 * U) {
        uint2 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = *reinterpret_cast<const uint2*>(X + (long long)min(t + 64 * u, n - 1) * K + kk);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            xm[0] = fmaxf(xm[0], fabsf(in2f<DT>(v[u].x & 0xFFFFu)));
            xm[1] = fmaxf(xm[1], fabsf(in2f<DT>(v[u].x >> 16)));
            xm[2] = fmaxf(xm[2], fabsf(in2f<DT>(v[u].y & 0xFFFFu)));
            xm[3] = fmaxf(xm[3], fabsf(in2f<DT>(v[u].y >> 16)));
        }
    }
    for (int r = rg; r < N; r += 64 * U) {
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = *reinterpret_cast<const float4*>(W + (long long)min(r + 64 * u, N - 1) * K + kk);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            wm[0] = fmaxf(wm[0], fabsf(v[u].x));
            wm[1] = fmaxf(wm[1], fabsf(v[u].y));
            wm[2] = fmaxf(wm[2], fabsf(v[u].z));
            wm[3] = fmaxf(wm[3], fabsf(v[u].w));
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        red[0][rg][4 * cg + j] = xm[j];
        red[1][rg][4 * cg + j] = wm[j];
    }
    __syncthreads();
    if (tid < 64) {
        const int k = blockIdx.x * 64 + tid;
        float x = 0.0f, w = 0.0f;
        for (int g = 0; g < 64; ++g) {
            x = fmaxf(x, red[0][g][tid]);
            w = fmaxf(w, red[1][g][tid]);
        }
        if (k < K) {
            const float num = pow_quarters(x, a);
            const float den = pow_quarters(w, 4 - a);
            const float v = num / (den == 0.0f ? 1.0f : den);
            s[k] = (x == 0.0f || w == 0.0f) ? 1.0f : v;
        }
    }
}

// Row-wise symmetric INT8: v = w * s_j (WEIGHT) or x / s_j; one workgroup per row.
template <int DT, bool WEIGHT>
__global__ __launch_bounds__(256) void quant_rows_kernel(const void* __restrict__ src, int K,
                                                         const float* __restrict__ s, int8_t* __restrict__ q,
                                                         float* __restrict__ scale) {
    __shared__ float red[256];
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    auto value = [&](int k) -> float {
        if constexpr (WEIGHT) return static_cast<const float*>(src)[(long long)row * K + k] * s[k];
        else return in2f<DT>(static_cast<const uint16_t*>(src)[(long long)row * K + k]) / s[k];
    };
    float amax = 0.0f;
    for (int k = tid; k < K; k += 256) amax = fmaxf(amax, fabsf(value(k)));
    red[tid] = amax;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
        __syncthreads();
    }
    float sc = red[0] / 127.0f;
    if (sc == 0.0f) sc = 1.0f;
    for (int k = tid; k < K; k += 256) {
        const float c = fminf(fmaxf(__builtin_rintf(value(k) / sc), -128.0f), 127.0f);
        q[(long long)row * K + k] = (int8_t)(int)c;
    }
    if (tid == 0) scale[row] = sc;
}

// Vectorized variant for K % 8 == 0 and K <= 8 * 256 * CH: thread t holds chunks t + 256 c
// (8 consecutive values each) in registers between the max and the code pass; same
// arithmetic as quant_rows_kernel.
template <int DT, bool WEIGHT, int CH>
__global__ __launch_bounds__(256) void quant_rows_vec_kernel(const void* __restrict__ src, int K,
                                                             const float* __restrict__ s, int8_t* __restrict__ q,
                                                             float* __restrict__ scale) {
    __shared__ float red[256];
    const int row = blockIdx.x;
    const int tid = threadIdx.x;
    const int nch = K >> 3;
    float v[CH][8];
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int ch = tid + 256 * c;
        if (ch < nch) {
            const float4 s0 = *reinterpret_cast<const float4*>(s + 8 * ch);
            const float4 s1 = *reinterpret_cast<const float4*>(s + 8 * ch + 4);
            const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
            if constexpr (WEIGHT) {
                const float* p = static_cast<const float*>(src) + (long long)row * K + 8 * ch;
                const float4 a = *reinterpret_cast<const float4*>(p);
                const float4 b = *reinterpret_cast<const float4*>(p + 4);
                const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) v[c][i] = x[i] * sv[i];
            } else {
                const u32x4 r = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(src) + (long long)row * K + 8 * ch);
                const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) v[c][i] = in2f<DT>((w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu) / sv[i];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[c][i]));
        }
    }
    red[tid] = amax;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
        __syncthreads();
    }
    float sc = red[0] / 127.0f;
    if (sc == 0.0f) sc = 1.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int ch = tid + 256 * c;
        if (ch < nch) {
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float cq = fminf(fmaxf(__builtin_rintf(v[c][i] / sc), -128.0f), 127.0f);
                const uint32_t b = (uint32_t)(int)cq & 0xFFu;
                if (i < 4) lo |= b << (8 * i); else hi |= b << (8 * (i - 4));
            }
            *reinterpret_cast<uint2*>(q + (long long)row * K + 8 * ch) = make_uint2(lo, hi);
        }
    }
    if (tid == 0) scale[row] = sc;
}

constexpr int I_BM = 256, I_BN = 256, I_BK = 128;      // bytes of K per step
constexpr int kGemmLds = 4 * I_BM * 8 * 16;            // A and B, two buffers each: 128 KB

template <int DT>
__global__ __launch_bounds__(512, 1) void w8a8_gemm_kernel(const int8_t* __restrict__ qx, const float* __restrict__ sx,
                                                           const int8_t* __restrict__ qw, const float* __restrict__ sw,
                                                           uint16_t* __restrict__ Y, int M, int N, int K) {
    extern __shared__ __attribute__((aligned(16))) u32x4 lds8[];
    // buffers: A0, A1, B0, B1 of I_BM * 8 slots each
    auto As = [&](int b) { return lds8 + b * (I_BM * 8); };
    auto Bs = [&](int b) { return lds8 + (2 + b) * (I_BM * 8); };
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int h = lane >> 5;
    const int wm = wave >> 2, wn = wave & 3;
    int mt, nt;
    if (!xcd_tile(blockIdx.x, (M + I_BM - 1) / I_BM, (N + I_BN - 1) / I_BN, mt, nt)) return;
    const int m0 = mt * I_BM;
    const int n0 = nt * I_BN;
    const int nsteps = K / I_BK;

    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(qx), 0, 0x7FFFFFFF, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(qw), 0, 0x7FFFFFFF, 0x00020000);
    // instruction j of wave w fills slots (4 w + j) * 64 + lane: row r = (4 w + j) * 8 + lane / 8,
    // slot lane % 8 holding piece (lane % 8) ^ (r / 2 % 8); rows past M / N are clamped
    int aoff[4], boff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = (4 * wave + j) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        aoff[j] = min(m0 + r, M - 1) * K + 16 * c;
        boff[j] = min(n0 + r, N - 1) * K + 16 * c;
    }
    auto load = [&](int buf, int step) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (__attribute__((address_space(3))) void*)(As(buf) + (4 * wave + j) * 64), 16, aoff[j], step * I_BK, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (__attribute__((address_space(3))) void*)(Bs(buf) + (4 * wave + j) * 64), 16, boff[j], step * I_BK, 0, 0);
        }
    };
    // fragment slots: tile row rr = 32 t + l32, piece 4 h + j -> slot rr * 8 + ((4 h + j) ^ (rr / 2 % 8))
    int fslot[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) fslot[j] = l32 * 8 + ((4 * h + j) ^ ((l32 >> 1) & 7));

    v16i acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jn = 0; jn < 2; ++jn)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][jn][e] = 0;

    auto compute = [&](int buf) {
        const u32x4* A = As(buf) + wm * 128 * 8;
        const u32x4* B = Bs(buf) + wn * 64 * 8;
        u32x4 fa[2][4], fb[2][2];
#pragma unroll
        for (int t = 0; t < 4; ++t) fa[0][t] = A[t * 256 + fslot[0]];
#pragma unroll
        for (int t = 0; t < 2; ++t) fb[0][t] = B[t * 256 + fslot[0]];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int cur = j & 1;
            if (j < 3) {
#pragma unroll
                for (int t = 0; t < 4; ++t) fa[cur ^ 1][t] = A[t * 256 + fslot[j + 1]];
#pragma unroll
                for (int t = 0; t < 2; ++t) fb[cur ^ 1][t] = B[t * 256 + fslot[j + 1]];
            }
#pragma unroll
            for (int tm = 0; tm < 4; ++tm) {
                const v4i av = __builtin_bit_cast(v4i, fa[cur][tm]);
#pragma unroll
                for (int tn = 0; tn < 2; ++tn)
                    acc[tm][tn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, __builtin_bit_cast(v4i, fb[cur][tn]),
                                                                        acc[tm][tn], 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (j < 3) {
                    if (i < 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // DS read
                    else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                  // MFMA
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    load(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int step = 0; step < nsteps; ++step) {
        const int buf = step & 1;
        if (step + 1 < nsteps) load(buf ^ 1, step + 1);
        compute(buf);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    // epilogue: lane (l32, h) element e of tile (tm, tn) is row 32 tm + 8 (e / 4) + 4 h + e % 4,
    // column 32 tn + l32 of the wave's 128 x 64
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) {
        const int n = n0 + wn * 64 + tn * 32 + l32;
        if (n >= N) continue;
        const float swn = sw[n];
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = m0 + wm * 128 + tm * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
                if (m < M) {
                    // two fp32 roundings, then one to 16 bits: the empty asm keeps the
                    // compiler from fusing the last multiply into the conversion
                    float y = ((float)acc[tm][tn][e] * sx[m]) * swn;
                    asm volatile("" : "+v"(y));
                    Y[(long long)m * N + n] = f2out<DT>(y);
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_w8a8_smooth(const void* X, int dtype, int n, const float* W, int N, int K, int a, float* s,
                              hipStream_t st) {
    const auto x = static_cast<const uint16_t*>(X);
    if (K % 4 == 0 && (reinterpret_cast<uintptr_t>(X) & 7) == 0 && (reinterpret_cast<uintptr_t>(W) & 15) == 0) {
        const dim3 grid((K + 63) / 64);
        if (dtype == DT_F16)
            hipLaunchKernelGGL(smooth_tile_kernel<DT_F16>, grid, dim3(1024), 0, st, x, n, W, N, K, a, s);
        else
            hipLaunchKernelGGL(smooth_tile_kernel<DT_BF16>, grid, dim3(1024), 0, st, x, n, W, N, K, a, s);
        return hipGetLastError();
    }
    const dim3 grid((K + 255) / 256);
    if (dtype == DT_F16)
        hipLaunchKernelGGL(smooth_kernel<DT_F16>, grid, dim3(256), 0, st, x, n, W, N, K, a, s);
    else
        hipLaunchKernelGGL(smooth_kernel<DT_BF16>, grid, dim3(256), 0, st, x, n, W, N, K, a, s);
    return hipGetLastError();
}

namespace {

// vectorized rows when every pointer and row is 16-byte aligned and a row fits 8 chunks per
// thread; the scalar kernel otherwise (same arithmetic)
template <int DT, bool WEIGHT>
hipError_t quant_rows(const void* src, int R, int K, const float* s, int8_t* q, float* scale, hipStream_t st) {
    const bool vec = K % 16 == 0 && K <= 8 * 256 * 8 && (reinterpret_cast<uintptr_t>(src) & 15) == 0 &&
                     (reinterpret_cast<uintptr_t>(s) & 15) == 0 && (reinterpret_cast<uintptr_t>(q) & 7) == 0;
    if (!vec) {
        hipLaunchKernelGGL((quant_rows_kernel<DT, WEIGHT>), dim3(R), dim3(256), 0, st, src, K, s, q, scale);
    } else if (K <= 8 * 256 * 2) {
        hipLaunchKernelGGL((quant_rows_vec_kernel<DT, WEIGHT, 2>), dim3(R), dim3(256), 0, st, src, K, s, q, scale);
    } else if (K <= 8 * 256 * 4) {
        hipLaunchKernelGGL((quant_rows_vec_kernel<DT, WEIGHT, 4>), dim3(R), dim3(256), 0, st, src, K, s, q, scale);
    } else {
        hipLaunchKernelGGL((quant_rows_vec_kernel<DT, WEIGHT, 8>), dim3(R), dim3(256), 0, st, src, K, s, q, scale);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_w8a8_quant_weight(const float* W, int N, int K, const float* s, int8_t* q, float* sw, hipStream_t st) {
    return quant_rows<DT_F16, true>(W, N, K, s, q, sw, st);
}

hipError_t launch_w8a8_quant_act(const void* X, int dtype, int M, int K, const float* s, int8_t* q, float* sx,
                                 hipStream_t st) {
    return dtype == DT_F16 ? quant_rows<DT_F16, false>(X, M, K, s, q, sx, st)
                           : quant_rows<DT_BF16, false>(X, M, K, s, q, sx, st);
}

hipError_t launch_w8a8_linear(const int8_t* qx, const float* sx, int M, int N, int K, const int8_t* qw,
                              const float* sw, void* Y, int dtype, hipStream_t st) {
    const int tiles = ((M + I_BM - 1) / I_BM) * ((N + I_BN - 1) / I_BN);
    const int grid = 8 * ((tiles + 7) / 8);
    // 128 KB of LDS per block (the default limit is 64 KB); set on every launch
    const void* fn = dtype == DT_F16 ? reinterpret_cast<const void*>(&w8a8_gemm_kernel<DT_F16>)
                                     : reinterpret_cast<const void*>(&w8a8_gemm_kernel<DT_BF16>);
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds);
    if (e != hipSuccess) return e;
    if (dtype == DT_F16)
        hipLaunchKernelGGL(w8a8_gemm_kernel<DT_F16>, dim3(grid), dim3(512), kGemmLds, st, qx, sx, qw, sw,
                           static_cast<uint16_t*>(Y), M, N, K);
    else
        hipLaunchKernelGGL(w8a8_gemm_kernel<DT_BF16>, dim3(grid), dim3(512), kGemmLds, st, qx, sx, qw, sw,
                           static_cast<uint16_t*>(Y), M, N, K);
    return hipGetLastError();
}

}  // namespace w4a16
