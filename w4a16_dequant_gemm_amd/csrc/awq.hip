// AWQ on the GPU: the per-channel activation statistic, the grid search over channel
// scalings with the quantized layer's output error, and the scaling of activations.
//
// Method (page "推理优化中“用精度换性能“的核心技术：量化", section 五 AWQ): a channel's
// importance follows its mean activation magnitude on calibration data (5.1); the layer is
// rescaled exactly, W x = (W diag(1/s)) (diag(s) x), so the quantizer sees W / s (5.2); the
// scale vector is the candidate whose quantized layer has the smallest output error on the
// calibration data (5.2, grid search); the quantizer is the plain group-wise RTN (5.3).
// Candidates: s = r^(a/4), a = -4 .. 4, r the statistic normalized to a geometric centre of
// 1 (clamped at 1e-6 of its maximum); every candidate comes from IEEE fp32 square roots,
// products and one division, so it is reproducible bit for bit, and so are the codes of
// W / s.  The output error of candidate a is ||X E^T||_F^2 with E = W - s * W_hat' (fp64):
// one fp64 GEMM (X [n, K] times E^T) and a fixed-order sum of squares per candidate.  The
// best index is chosen on the device (first minimum), so the whole search is one
// asynchronous sequence of launches.
#include "common.h"
#include "gemm_f64.h"
#include "launch.h"

namespace w4a16 {

namespace {

constexpr int kGrid = 9;                 // exponents a / 4, a = -4 .. 4
constexpr int kPartials = 1024;          // blocks of the sum of squares

template <int DT>
__global__ __launch_bounds__(256) void awq_stats_kernel(const uint16_t* __restrict__ X, int n, int K,
                                                        float* __restrict__ xmean) {
    const int k = blockIdx.x * 256 + threadIdx.x;
    if (k >= K) return;
    double s = 0.0;
    for (int t = 0; t < n; ++t) s += fabs((double)in2f<DT>(X[(long long)t * K + k]));
    xmean[k] = (float)(s / (double)n);
}

// S[a][k] for the nine exponents (one workgroup; K <= 2^31)
__global__ __launch_bounds__(1024) void awq_candidates_kernel(const float* __restrict__ xmean, int K,
                                                              float* __restrict__ S) {
    __shared__ float red[1024];
    const int tid = threadIdx.x;
    float mx = 0.0f;
    for (int k = tid; k < K; k += 1024) mx = fmaxf(mx, xmean[k]);
    red[tid] = mx;
    __syncthreads();
    for (int w = 512; w > 0; w >>= 1) {
        if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
        __syncthreads();
    }
    mx = red[0];
    __syncthreads();
    const float lo = 1e-6f * mx;
    float mn = __builtin_inff();
    for (int k = tid; k < K; k += 1024) mn = fminf(mn, fmaxf(xmean[k], lo));
    red[tid] = mn;
    __syncthreads();
    for (int w = 512; w > 0; w >>= 1) {
        if (tid < w) red[tid] = fminf(red[tid], red[tid + w]);
        __syncthreads();
    }
    mn = red[0];
    const float norm = sqrtf(mx * mn);
    for (int k = tid; k < K; k += 1024) {
        const float r = fmaxf(xmean[k], lo) / norm;
        const float q = sqrtf(sqrtf(r));
        float p = 1.0f;
        S[4 * K + k] = 1.0f;
        for (int a = 1; a <= 4; ++a) {
            p = p * q;
            S[(4 + a) * K + k] = p;
            S[(4 - a) * K + k] = 1.0f / p;
        }
    }
}

// RTN of W / s per group (lanes own whole 32-bit words; `seg` lanes per group), writing
// the fp64 error E = W - s * W_hat' and, when OUT, the packed result.  `best` (device)
// selects the candidate row of S when OUT; else `a` does.
template <int SCHEME, bool OUT>
__global__ __launch_bounds__(256) void awq_quant_kernel(const float* __restrict__ W, int N, int K, int g, int G,
                                                        int seg, int words_per_lane, const float* __restrict__ S,
                                                        int a, const int* __restrict__ best,
                                                        double* __restrict__ E, uint32_t* __restrict__ qw,
                                                        uint16_t* __restrict__ scales, uint16_t* __restrict__ zeros,
                                                        float* __restrict__ s_out) {
    const int lane = threadIdx.x & 63;
    const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int gpw = 64 / seg;
    const int slot = lane / seg;
    const int gl = lane % seg;
    const long long gid = (long long)wave * gpw + slot;
    const bool active = gid < (long long)N * G;
    const int n = active ? (int)(gid / G) : 0;
    const int j = active ? (int)(gid % G) : 0;
    const int wcount = g >> 3;
    const float* s = S + (long long)(OUT ? *best : a) * K + (long long)j * g;
    const float* row = W + (long long)n * K + (long long)j * g;
    float mn = __builtin_inff(), mx = -__builtin_inff();
    for (int it = 0; it < words_per_lane; ++it) {
        const int w = gl + it * seg;
        if (active && w < wcount) {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float x = row[8 * w + t] / s[8 * w + t];
                if (SCHEME == 0) { mn = fminf(mn, x); mx = fmaxf(mx, x); }
                else mx = fmaxf(mx, fabsf(x));
            }
        }
    }
    for (int off = seg >> 1; off > 0; off >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, off, 64));
        mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    }
    if (!active) return;
    _Float16 sh;
    float sc, z;
    rtn_params<SCHEME>(mn, mx, sh, sc, z);
    for (int it = 0; it < words_per_lane; ++it) {
        const int w = gl + it * seg;
        if (w < wcount) {
            uint32_t word = 0;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int k = 8 * w + t;
                const float wv = row[k];
                const uint32_t q = rtn_code<SCHEME>(wv / s[k], sc, z);
                word |= (q & 0xFu) << (4 * t);
                if (!OUT) {
                    const double what = (double)sc * ((double)q - (double)z);
                    E[(long long)n * K + (long long)j * g + k] = (double)wv - (double)s[k] * what;
                }
            }
            if (OUT) qw[(long long)n * (K >> 3) + (long long)j * (g >> 3) + w] = word;
        }
    }
    if (OUT && gl == 0) {
        scales[(long long)n * G + j] = __builtin_bit_cast(uint16_t, sh);
        if (zeros) zeros[(long long)n * G + j] = __builtin_bit_cast(uint16_t, (_Float16)z);
    }
    if (OUT && n == 0 && gl == 0) {
        // row 0's groups publish the chosen scale vector
        for (int k = 0; k < g; ++k) s_out[(long long)j * g + k] = s[k];
    }
}

// fixed-order sum of squares: per-block partials, then one block adds them in order
__global__ __launch_bounds__(256) void sumsq_partial_kernel(const double* __restrict__ D, long long len,
                                                            double* __restrict__ part) {
    __shared__ double red[256];
    double s = 0.0;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < len; i += (long long)gridDim.x * 256)
        s = fma(D[i], D[i], s);
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(256) void sumsq_final_kernel(const double* __restrict__ part, int nparts,
                                                          double* __restrict__ out) {
    __shared__ double red[256];
    double s = 0.0;
    for (int i = threadIdx.x; i < nparts; i += 256) s += part[i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) *out = red[0];
}

__global__ void argmin_kernel(const double* __restrict__ losses, int count, int* __restrict__ best) {
    if (threadIdx.x != 0) return;
    int b = 0;
    for (int i = 1; i < count; ++i)
        if (losses[i] < losses[b]) b = i;
    *best = b;
}

// x * s per channel rounded once to the 16-bit dtype: the fp64 product is exact; it is
// rounded to fp32 with round-to-odd (truncate, then set the last bit if inexact), which
// makes the following round-to-nearest-even to 16 bits a single correct rounding.
template <int DT>
__global__ __launch_bounds__(256) void awq_scale_kernel(const uint16_t* __restrict__ X, long long total, int K,
                                                        const float* __restrict__ s, uint16_t* __restrict__ Y) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const double p = (double)in2f<DT>(X[i]) * (double)s[i % K];
    float f = (float)p;
    if ((double)f != p) {
        if (fabs((double)f) > fabs(p)) f = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, f) - 1u);
        f = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, f) | 1u);
    }
    Y[i] = f2out<DT>(f);
}

}  // namespace

long long awq_workspace_doubles(long long N, long long K, long long n) {
    return N * K + n * N + kPartials + (kGrid * K + 1) / 2 + 2;
}

hipError_t launch_awq_stats(const void* X, int dtype, int n, int K, float* xmean, hipStream_t st) {
    const dim3 grid((K + 255) / 256);
    if (dtype == DT_F16)
        hipLaunchKernelGGL(awq_stats_kernel<DT_F16>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(X), n,
                           K, xmean);
    else
        hipLaunchKernelGGL(awq_stats_kernel<DT_BF16>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(X),
                           n, K, xmean);
    return hipGetLastError();
}

hipError_t launch_awq_search(const float* W, int N, int K, const void* X, int dtype, int n, const float* xmean,
                             int g, int scheme, double* work, double* losses, int* best, float* s_out,
                             uint32_t* qw, uint16_t* scales, uint16_t* zeros, hipStream_t st) {
    double* E = work;
    double* D = E + (long long)N * K;
    double* part = D + (long long)n * N;
    float* S = reinterpret_cast<float*>(part + kPartials);
    hipLaunchKernelGGL(awq_candidates_kernel, dim3(1), dim3(1024), 0, st, xmean, K, S);
    const int G = K / g;
    const int wcount = g / 8;
    const bool pow2 = (wcount & (wcount - 1)) == 0;
    const int seg = (pow2 && wcount <= 64) ? wcount : 64;
    const int wpl = (wcount + seg - 1) / seg;
    const long long waves = ((long long)N * G + (64 / seg) - 1) / (64 / seg);
    const unsigned qblocks = (unsigned)((waves + 3) / 4);
    const long long dlen = (long long)n * N;
    for (int a = 0; a < kGrid; ++a) {
        if (scheme == 0)
            hipLaunchKernelGGL((awq_quant_kernel<0, false>), dim3(qblocks), dim3(256), 0, st, W, N, K, g, G, seg,
                               wpl, S, a, best, E, qw, scales, zeros, s_out);
        else
            hipLaunchKernelGGL((awq_quant_kernel<1, false>), dim3(qblocks), dim3(256), 0, st, W, N, K, g, G, seg,
                               wpl, S, a, best, E, qw, scales, zeros, s_out);
        // D = X E^T: A(m, k) = X[m][k], B(k, j) = E[j][k]
        const hipError_t e = dtype == DT_F16
                                 ? gemm<1, 0, 0>(n, N, K, 1.0, X, K, 1, E, 1, K, 0.0, D, N, 1, st)
                                 : gemm<2, 0, 0>(n, N, K, 1.0, X, K, 1, E, 1, K, 0.0, D, N, 1, st);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(sumsq_partial_kernel, dim3(kPartials), dim3(256), 0, st, D, dlen, part);
        hipLaunchKernelGGL(sumsq_final_kernel, dim3(1), dim3(256), 0, st, part, kPartials, losses + a);
    }
    hipLaunchKernelGGL(argmin_kernel, dim3(1), dim3(64), 0, st, losses, kGrid, best);
    if (scheme == 0)
        hipLaunchKernelGGL((awq_quant_kernel<0, true>), dim3(qblocks), dim3(256), 0, st, W, N, K, g, G, seg, wpl,
                           S, 0, best, E, qw, scales, zeros, s_out);
    else
        hipLaunchKernelGGL((awq_quant_kernel<1, true>), dim3(qblocks), dim3(256), 0, st, W, N, K, g, G, seg, wpl,
                           S, 0, best, E, qw, scales, zeros, s_out);
    return hipGetLastError();
}

hipError_t launch_awq_scale(const void* X, int dtype, long long M, int K, const float* s, void* Y,
                            hipStream_t st) {
    const long long total = M * K;
    const dim3 grid((unsigned)((total + 255) / 256));
    if (dtype == DT_F16)
        hipLaunchKernelGGL(awq_scale_kernel<DT_F16>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(X), total,
                           K, s, static_cast<uint16_t*>(Y));
    else
        hipLaunchKernelGGL(awq_scale_kernel<DT_BF16>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(X),
                           total, K, s, static_cast<uint16_t*>(Y));
    return hipGetLastError();
}

}  // namespace w4a16
