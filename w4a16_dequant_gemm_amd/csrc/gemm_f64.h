// fp64 GEMM over strided operands (used by the GPTQ and AWQ calibration steps).
#pragma once

#include "common.h"

namespace w4a16 {

constexpr int GT = 64;      // tile edge
constexpr int GKC = 16;     // k chunk

// element loaders: 0 = fp64, 1 = fp16 bits, 2 = bf16 bits
template <int T>
__device__ __forceinline__ double ld_elem(const void* p, long long i) {
    if constexpr (T == 0) return static_cast<const double*>(p)[i];
    else if constexpr (T == 1) return (double)h2f(static_cast<const uint16_t*>(p)[i]);
    else return (double)bf2f(static_cast<const uint16_t*>(p)[i]);
}

// C = beta * C + alpha * A B with A(m, k) = A[m sam + k sak], B(k, n) = B[k sbk + n sbn],
// C(m, n) = C[m scm + n scn].  MODE bit 0: only tiles touching the lower triangle
// (m >= n) are computed; bit 1: B is lower triangular (B(k, n) = 0 for k < n): the
// contraction of a tile starts at its first column and the strictly upper entries are read
// as zeros whatever memory holds there; bit 2: A is lower triangular (A(m, k) = 0 for
// k > m): it ends after the tile's last row, strictly upper entries read as zeros.
// beta == 0 never reads C.
template <int AT, int BT, int MODE>
__global__ __launch_bounds__(256) void gemm_f64_kernel(int M, int N, int K, double alpha,
                                                       const void* __restrict__ A, long long sam,
                                                       long long sak, const void* __restrict__ B,
                                                       long long sbk, long long sbn, double beta,
                                                       double* __restrict__ C, long long scm,
                                                       long long scn) {
    const int m0 = blockIdx.y * GT;
    const int n0 = blockIdx.x * GT;
    if ((MODE & 1) && n0 > m0 + GT - 1) return;
    __shared__ double As[GKC][GT + 1];
    __shared__ double Bs[GKC][GT + 1];
    const int tid = threadIdx.x;
    const int tx = tid & 15;
    const int ty = tid >> 4;
    double acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
    const int kbeg = (MODE & 2) ? (n0 / GKC) * GKC : 0;
    const int kend = (MODE & 4) ? min(K, m0 + GT) : K;
    const bool a_krow = sak == 1;      // k contiguous in A
    const bool b_ncol = sbn == 1;      // n contiguous in B
    for (int k0 = kbeg; k0 < kend; k0 += GKC) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = tid + 256 * r;
            int m, k;
            if (a_krow) { m = e >> 4; k = e & 15; } else { k = e >> 6; m = e & 63; }
            const int gm = m0 + m, gk = k0 + k;
            As[k][m] = (gm < M && gk < K && (!(MODE & 4) || gk <= gm))
                           ? ld_elem<AT>(A, (long long)gm * sam + (long long)gk * sak) : 0.0;
            int n, kb;
            if (b_ncol) { kb = e >> 6; n = e & 63; } else { n = e >> 4; kb = e & 15; }
            const int gn = n0 + n, gkb = k0 + kb;
            Bs[kb][n] = (gn < N && gkb < K && (!(MODE & 2) || gkb >= gn))
                            ? ld_elem<BT>(B, (long long)gkb * sbk + (long long)gn * sbn) : 0.0;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < GKC; ++kk) {
            double a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int gm = m0 + ty + 16 * i, gn = n0 + tx + 16 * j;
            if (gm < M && gn < N) {
                double* c = C + (long long)gm * scm + (long long)gn * scn;
                *c = beta == 0.0 ? alpha * acc[i][j] : fma(alpha, acc[i][j], beta * *c);
            }
        }
}

template <int AT, int BT, int MODE>
hipError_t gemm(int M, int N, int K, double alpha, const void* A, long long sam, long long sak,
                const void* B, long long sbk, long long sbn, double beta, double* C, long long scm,
                long long scn, hipStream_t st) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const dim3 grid((N + GT - 1) / GT, (M + GT - 1) / GT);
    hipLaunchKernelGGL((gemm_f64_kernel<AT, BT, MODE>), grid, dim3(256), 0, st, M, N, K, alpha, A, sam,
                       sak, B, sbk, sbn, beta, C, scm, scn);
    return hipGetLastError();
}

}  // namespace w4a16
