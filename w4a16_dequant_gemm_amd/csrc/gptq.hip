// GPTQ on the GPU: the layer Hessian from calibration activations, the Cholesky factor of
// its (damped) inverse, and the column-by-column INT4 quantization with second-order
// compensation of the columns not yet quantized.
//
// Method (page "推理优化中“用精度换性能“的核心技术：量化", section 四 GPTQ, 4.2 and 4.4):
// H = 2 X^T X; columns are quantized in their natural order; after column i the columns
// j > i move by -dw * Hinv[i, j] / Hinv[i, i], Hinv being the inverse Hessian of the columns
// still free.  With H^-1 = U^T U (U upper triangular) that ratio is U[i, j] / U[i, i], so
// the loop needs only the rows of U (the Cholesky factor the page mentions).  Group
// parameters are the RTN ones of the group's current weights when the loop reaches the
// group's first column.  Everything but the code decision (fp32 RTN, as in quantize.hip)
// is fp64.
//
// GPU structure.
//   * fp64 GEMM (64 x 64 tiles, 16-deep k chunks through LDS, 4 x 4 outputs per thread)
//     over strided operands: the Hessian, the Cholesky trailing updates, the triangular
//     inverse and the GPTQ batch updates are all instances of it.
//   * U without an explicit inverse of H: with P the index reversal, P H P = L L^T
//     (lower Cholesky) gives H = (P L P)(P L P)^T, so U = P L^-1 P.  The matrix is
//     reversed once, factored by blocks of 64 (one-workgroup diagonal factorization and
//     inverse, a row-parallel panel solve, a lower-tile GEMM for the trailing matrix),
//     L^-1 is built block row by block row from GEMMs, and reversed back into U.
//   * The column loop runs in batches of B = 64 (or 32) columns: one lane per weight row
//     holds the batch in registers and applies the in-batch compensation sequentially; the
//     batch's scaled errors then update all later columns in one GEMM (the order of the
//     additions changes, the arithmetic does not).
#include "common.h"
#include "gemm_f64.h"
#include "launch.h"

namespace w4a16 {

namespace {

// ------------------------------------------------- damping, reversal, Cholesky
// lambda = damp * mean(diag H), stored in H[0][1] (strictly upper: never read as data)
__global__ __launch_bounds__(1024) void damp_kernel(double* H, long long K, double damp) {
    __shared__ double part[1024];
    double s = 0.0;
    for (long long i = threadIdx.x; i < K; i += 1024) s += H[i * K + i];
    part[threadIdx.x] = s;
    __syncthreads();
    for (int w = 512; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) H[1] = damp * (part[0] / (double)K);
}

// dst[i][j] = src[K-1-i][K-1-j], reading only the lower triangle of the symmetric src;
// DAMP adds lambda (src[0][1]) on the diagonal; UPPER_OUT zeroes dst below the diagonal.
template <bool DAMP, bool UPPER_OUT>
__global__ __launch_bounds__(256) void reverse_kernel(const double* __restrict__ src, double* __restrict__ dst,
                                                      long long K) {
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= K * K) return;
    const long long i = idx / K, j = idx % K;
    if (UPPER_OUT && j < i) { dst[idx] = 0.0; return; }
    long long a = K - 1 - i, b = K - 1 - j;
    if (b > a) { const long long t = a; a = b; b = t; }
    double v = src[a * K + b];
    if (DAMP && i == j) v += src[1];
    dst[idx] = v;
}

// One diagonal block (jb <= 64) of the lower Cholesky factorization, in place, by one
// workgroup; its inverse (lower, zeros above the diagonal) goes to Dinv.  Thread t owns
// row i = t / 4, columns 16 (t % 4) .. + 15 of the block in registers for both
// right-looking sweeps; the pivot column (Cholesky) or pivot row (inverse) of each step is
// published through LDS (double-buffered: one barrier per step).  The updates are
// branch-free: a zero multiplier leaves an element exactly as it is.  Rows and columns
// past jb hold the identity, which factors and inverts to itself.
__global__ __launch_bounds__(256) void potrf_diag_kernel(double* __restrict__ A, long long lda, int jb,
                                                         double* __restrict__ Dinv, long long ldd) {
    __shared__ double col[2][64];
    __shared__ double L[64][65];
    __shared__ double rdiag[64];
    const int tid = threadIdx.x;
    const int i = tid >> 2;
    const int q = tid & 3;
    double r[16];
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
        const int j = q * 16 + jj;
        r[jj] = (i < jb && j < jb) ? A[(long long)i * lda + j] : (i == j ? 1.0 : 0.0);
    }
    // Cholesky: l_k = a[:, k] / sqrt(a[k][k]); a[i][j] -= l_i l_j for k < j <= i
    for (int kq = 0; kq < 4; ++kq) {
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            const int k = kq * 16 + kk;
            const int buf = k & 1;
            if (q == kq) col[buf][i] = r[kk];
            __syncthreads();
            const double d = sqrt(col[buf][k]);
            const double rd = 1.0 / d;
            const double li = i == k ? d : (i > k ? col[buf][i] * rd : 0.0);
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                const int j = q * 16 + jj;
                const double lj = (j > k && j <= i) ? col[buf][j] * rd : 0.0;
                r[jj] = fma(-li, lj, r[jj]);
            }
            if (q == kq && i >= k) r[kk] = li;
        }
    }
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) L[i][q * 16 + jj] = r[jj];
    __syncthreads();
    if (tid < 64) rdiag[tid] = 1.0 / L[tid][tid];
    // inverse: X = I; row k *= 1 / L[k][k]; rows i > k -= L[i][k] * row k
    double x[16];
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) x[jj] = (i == q * 16 + jj) ? 1.0 : 0.0;
    __syncthreads();
    for (int k = 0; k < 64; ++k) {
        const int buf = k & 1;
        if (i == k) {
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) {
                x[jj] *= rdiag[k];
                col[buf][q * 16 + jj] = x[jj];
            }
        }
        __syncthreads();
        const double lik = i > k ? L[i][k] : 0.0;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) x[jj] = fma(-lik, col[buf][q * 16 + jj], x[jj]);
    }
    if (i < jb) {
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
            const int j = q * 16 + jj;
            if (j < jb) {
                if (j <= i) A[(long long)i * lda + j] = r[jj];
                Dinv[(long long)i * ldd + j] = j <= i ? x[jj] : 0.0;
            }
        }
    }
}

// Panel solve, 16 rows per workgroup: row <- row * Dinv^T (Dinv lower, jb <= 64).
__global__ __launch_bounds__(256) void trsm_rows_kernel(double* __restrict__ A, long long lda, int rows, int jb,
                                                        const double* __restrict__ Dinv, long long ldd) {
    __shared__ double d[64][65];
    __shared__ double r[16][65];
    const int tid = threadIdx.x;
    const int row0 = blockIdx.x * 16;
    for (int e = tid; e < jb * jb; e += 256) d[e / jb][e % jb] = Dinv[(long long)(e / jb) * ldd + e % jb];
    for (int e = tid; e < 16 * jb; e += 256) {
        const int rr = e / jb, k = e % jb;
        r[rr][k] = row0 + rr < rows ? A[(long long)(row0 + rr) * lda + k] : 0.0;
    }
    __syncthreads();
    const int rr = tid >> 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = (tid & 15) + 16 * q;
        if (c < jb && row0 + rr < rows) {
            double x = 0.0;
            for (int k = 0; k <= c; ++k) x = fma(r[rr][k], d[c][k], x);
            A[(long long)(row0 + rr) * lda + c] = x;
        }
    }
}

// ------------------------------------------------------------- column loop
__global__ __launch_bounds__(256) void to_f64_kernel(const float* __restrict__ W, double* __restrict__ Wd,
                                                     long long n) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) Wd[i] = (double)W[i];
}

// RTN parameters of group [c0, c0 + g) of every row from the current weights (fp32).
template <int SCHEME>
__global__ __launch_bounds__(256) void group_params_kernel(const double* __restrict__ Wd, int N, int K,
                                                           int c0, int g, int G, uint16_t* __restrict__ scales,
                                                           uint16_t* __restrict__ zeros) {
    const int lane = threadIdx.x & 63;
    const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= N) return;
    const double* row = Wd + (long long)n * K + c0;
    float mn = __builtin_inff(), mx = -__builtin_inff();
    for (int k = lane; k < g; k += 64) {
        const float x = (float)row[k];
        if (SCHEME == 0) { mn = fminf(mn, x); mx = fmaxf(mx, x); }
        else mx = fmaxf(mx, fabsf(x));
    }
    for (int off = 32; off > 0; off >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, off, 64));
        mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    }
    if (lane == 0) {
        _Float16 sh;
        float s, z;
        rtn_params<SCHEME>(mn, mx, sh, s, z);
        scales[(long long)n * G + c0 / g] = __builtin_bit_cast(uint16_t, sh);
        if (zeros) zeros[(long long)n * G + c0 / g] = __builtin_bit_cast(uint16_t, (_Float16)z);
    }
}

// One batch of B columns [c0, c0 + B) (inside one group).  Four lanes share a weight row,
// lane q of the quad holding columns q B/4 .. + B/4 - 1 in registers.  For each column the
// owning lane decides the code and the error scaled by 1 / U[i][i], the quad takes it by a
// DPP broadcast, and every lane compensates its later columns.  The scaled errors go to E
// for the GEMM that updates the columns after the batch.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)0, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp((int)0, (int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

template <int B, int SCHEME>
__global__ __launch_bounds__(256) void gptq_batch_kernel(double* __restrict__ Wd, const double* __restrict__ U,
                                                         int N, int K, int c0, int g, int G,
                                                         const uint16_t* __restrict__ scales,
                                                         const uint16_t* __restrict__ zeros,
                                                         uint32_t* __restrict__ qw, double* __restrict__ E) {
    constexpr int Q = B / 4;            // columns per lane
    __shared__ double Us[B][B + 1];
    __shared__ double rinv[B];
    const int tid = threadIdx.x;
    for (int e = tid; e < B * B; e += 256) {           // strictly upper part only
        const int i = e / B, j = e % B;
        Us[i][j] = j > i ? U[(long long)(c0 + i) * K + c0 + j] : 0.0;
    }
    if (tid < B) rinv[tid] = 1.0 / U[(long long)(c0 + tid) * K + c0 + tid];
    __syncthreads();
    const int q = tid & 3;
    const int n_raw = blockIdx.x * 64 + (tid >> 2);
    const bool live = n_raw < N;
    const int n = live ? n_raw : N - 1;            // dead rows compute, never store
    double* row = Wd + (long long)n * K + c0 + q * Q;
    double w[Q], eown[Q];
#pragma unroll
    for (int j = 0; j < Q; ++j) w[j] = row[j];
    const int grp = c0 / g;
    const float s = h2f(scales[(long long)n * G + grp]);
    const float z = SCHEME == 0 ? h2f(zeros[(long long)n * G + grp]) : 8.0f;
    const double sd = (double)s, zd = (double)z;
    uint32_t words[Q / 8];
#pragma unroll
    for (int t = 0; t < Q / 8; ++t) words[t] = 0u;
    // column i = o Q + ii belongs to lane o of the quad; the (uniform) loop over o keeps
    // every register index static
    for (int o = 0; o < 4; ++o) {
#pragma unroll
        for (int ii = 0; ii < Q; ++ii) {
            const int i = o * Q + ii;
            // every lane evaluates its own column ii; only the owner's result is used
            const uint32_t qc = rtn_code<SCHEME>((float)w[ii], s, z);
            const double e_mine = (w[ii] - sd * ((double)qc - zd)) * rinv[i];
            double e;       // quad_perm broadcast of lane o
            switch (o) {
                case 0: e = dpp_f64<0x00>(e_mine); break;
                case 1: e = dpp_f64<0x55>(e_mine); break;
                case 2: e = dpp_f64<0xAA>(e_mine); break;
                default: e = dpp_f64<0xFF>(e_mine); break;
            }
            if (q == o) {
                words[ii / 8] |= (qc & 0xFu) << (4 * (ii % 8));
                eown[ii] = e;
            }
            // Us holds zeros on and below the diagonal: earlier columns stay exact
#pragma unroll
            for (int jj = 0; jj < Q; ++jj) w[jj] = fma(-e, Us[i][q * Q + jj], w[jj]);
        }
    }
    if (live) {
#pragma unroll
        for (int jj = 0; jj < Q; ++jj) E[(long long)n * B + q * Q + jj] = eown[jj];
#pragma unroll
        for (int t = 0; t < Q / 8; ++t) qw[(long long)n * (K / 8) + c0 / 8 + q * (Q / 8) + t] = words[t];
    }
}

template <int B, int SCHEME>
hipError_t gptq_loop(const float* W, int N, int K, int g, const double* U, double* Wd, double* E,
                     uint32_t* qw, uint16_t* scales, uint16_t* zeros, hipStream_t st) {
    const int G = K / g;
    const long long nk = (long long)N * K;
    hipLaunchKernelGGL(to_f64_kernel, dim3((unsigned)((nk + 255) / 256)), dim3(256), 0, st, W, Wd, nk);
    for (int c0 = 0; c0 < K; c0 += B) {
        if (c0 % g == 0)
            hipLaunchKernelGGL(group_params_kernel<SCHEME>, dim3((N + 3) / 4), dim3(256), 0, st, Wd, N, K, c0,
                               g, G, scales, SCHEME == 0 ? zeros : nullptr);
        hipLaunchKernelGGL((gptq_batch_kernel<B, SCHEME>), dim3((N + 63) / 64), dim3(256), 0, st, Wd, U, N,
                           K, c0, g, G, scales, zeros, qw, E);
        const int rest = K - c0 - B;
        if (rest > 0) {
            const hipError_t e = gemm<0, 0, 0>(N, rest, B, -1.0, E, B, 1, U + (long long)c0 * K + c0 + B, K, 1,
                                               1.0, Wd + c0 + B, K, 1, st);
            if (e != hipSuccess) return e;
        }
    }
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void fill_u16_kernel(uint16_t* __restrict__ p, long long n, uint16_t v) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_gptq_hessian(const void* X, int dtype, int n, int K, double* H, bool accumulate,
                               hipStream_t st) {
    // lower-triangle tiles of H (+)= 2 X^T X; A(m, k) = X[k][m], B(k, n) = X[k][n]
    const double beta = accumulate ? 1.0 : 0.0;
    if (dtype == DT_F16)
        return gemm<1, 1, 1>(K, K, n, 2.0, X, 1, K, X, K, 1, beta, H, K, 1, st);
    return gemm<2, 2, 1>(K, K, n, 2.0, X, 1, K, X, K, 1, beta, H, K, 1, st);
}

namespace {

// Inverse of the lower-triangular L (lower part of U) on the diagonal block [o, o + n), by
// halves: with L = [A 0; B C], L^-1 = [A^-1 0; -C^-1 B A^-1  C^-1].  A^-1 and C^-1 first
// (recursively; 64-blocks come from the diagonal factorization), then T = B A^-1, stored
// transposed in U's strictly upper part of the block, and -C^-1 T into H.
hipError_t trtri_lower(double* U, double* H, int K, int o, int n, hipStream_t st) {
    if (n <= 64) return hipSuccess;
    const int n1 = ((n / 2 + 63) / 64) * 64;
    const int n2 = n - n1;
    hipError_t e = trtri_lower(U, H, K, o, n1, st);
    if (e != hipSuccess) return e;
    e = trtri_lower(U, H, K, o + n1, n2, st);
    if (e != hipSuccess) return e;
    const long long lk = K;
    double* T = U + (long long)o * K + o + n1;          // T(m, n) at T[n K + m]
    e = gemm<0, 0, 2>(n2, n1, n1, 1.0, U + (long long)(o + n1) * K + o, lk, 1, H + (long long)o * K + o, lk, 1,
                      0.0, T, 1, lk, st);
    if (e != hipSuccess) return e;
    return gemm<0, 0, 4>(n2, n1, n2, -1.0, H + (long long)(o + n1) * K + o + n1, lk, 1, T, 1, lk, 0.0,
                         H + (long long)(o + n1) * K + o, lk, 1, st);
}

}  // namespace

hipError_t launch_gptq_factor(double* H, int K, double damp, double* U, hipStream_t st) {
    constexpr int NB = 64;
    const long long kk = (long long)K * K;
    const unsigned blocks = (unsigned)((kk + 255) / 256);
    // 1. lambda into H[0][1]; U = P (H + lambda I) P
    hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(1024), 0, st, H, (long long)K, damp);
    hipLaunchKernelGGL((reverse_kernel<true, false>), dim3(blocks), dim3(256), 0, st, H, U, (long long)K);
    // 2. lower Cholesky of U in place; the diagonal blocks' inverses go to H (block I, I)
    for (int j0 = 0; j0 < K; j0 += NB) {
        const int jb = min(NB, K - j0);
        double* Ajj = U + (long long)j0 * K + j0;
        double* Djj = H + (long long)j0 * K + j0;
        hipLaunchKernelGGL(potrf_diag_kernel, dim3(1), dim3(256), 0, st, Ajj, (long long)K, jb, Djj, (long long)K);
        const int rows = K - j0 - jb;
        if (rows > 0) {
            double* A21 = U + (long long)(j0 + jb) * K + j0;
            hipLaunchKernelGGL(trsm_rows_kernel, dim3((rows + 15) / 16), dim3(256), 0, st, A21, (long long)K, rows,
                               jb, Djj, (long long)K);
            const hipError_t e = gemm<0, 0, 1>(rows, rows, jb, -1.0, A21, K, 1, A21, 1, K, 1.0,
                                               U + (long long)(j0 + jb) * K + j0 + jb, K, 1, st);
            if (e != hipSuccess) return e;
        }
    }
    // 3. L^-1 in H (lower; the 64-blocks on the diagonal are already there)
    hipError_t e = trtri_lower(U, H, K, 0, K, st);
    if (e != hipSuccess) return e;
    // 4. U = P L^-1 P (upper; zeros below the diagonal)
    hipLaunchKernelGGL((reverse_kernel<false, true>), dim3(blocks), dim3(256), 0, st, H, U, (long long)K);
    return hipGetLastError();
}

hipError_t launch_gptq_quantize(const float* W, int N, int K, int g, int scheme, const double* U,
                                double* work, uint32_t* qw, uint16_t* scales, uint16_t* zeros,
                                hipStream_t st) {
    double* Wd = work;
    double* E = work + (long long)N * K;
    const bool b64 = g % 64 == 0 && K % 64 == 0;
    hipError_t e;
    if (scheme == 0)
        e = b64 ? gptq_loop<64, 0>(W, N, K, g, U, Wd, E, qw, scales, zeros, st)
                : gptq_loop<32, 0>(W, N, K, g, U, Wd, E, qw, scales, zeros, st);
    else
        e = b64 ? gptq_loop<64, 1>(W, N, K, g, U, Wd, E, qw, scales, zeros, st)
                : gptq_loop<32, 1>(W, N, K, g, U, Wd, E, qw, scales, zeros, st);
    if (e != hipSuccess) return e;
    if (scheme == 1 && zeros) {
        const long long n = (long long)N * (K / g);
        hipLaunchKernelGGL(fill_u16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, zeros, n,
                           (uint16_t)0x4800);
    }
    return hipGetLastError();
}

}  // namespace w4a16
