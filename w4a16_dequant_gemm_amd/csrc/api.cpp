// C ABI of the W4A16 library: argument validation, the M-based dispatcher and launches.
//
// Every check runs on the host before anything is enqueued, so invalid arguments never
// reach a kernel and never touch the GPU.  The dispatcher follows the regime split the
// pages draw: small batches (decode) are bound by reading the weights, large batches
// (prefill) by the matrix math (page "Quantization & Acceleration: 解释 W8A8 与 W4A16 的差异
// 与取舍", decode memory-bound / prefill compute-bound; page
// "大模型推理中 Weight-only、W8A8 和 FP8 量化有什么区别？如何选型？", sections 二 and 五).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <vector>

#include "../../include/w4a16.h"
#include "launch.h"

using w4a16::LinearArgs;

namespace {

constexpr int64_t kMaxDim = 2147483647LL;
constexpr int kMaxBatch = 65536;          // layers per w4a16_linear_batch call
constexpr int kGroupLaunch = 16;          // layers per grouped launch
constexpr int64_t kGptqMaxK = 46340;      // K * K fp64 elements indexable in 31 bits

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int log2_exact(int64_t v) {
    int s = 0;
    while ((int64_t(1) << s) < v) ++s;
    return (int64_t(1) << s) == v ? s : -1;
}

// Shape and group-size rules shared by all entry points.  On success fills g-derived
// fields (G, gshift).
int check_shape_group(int64_t N, int64_t K, int64_t g, int* G, int* gshift) {
    if (N < 1 || K < 1 || N > kMaxDim || K > kMaxDim) return W4A16_ERR_SHAPE;
    if (K % 32 != 0) return W4A16_ERR_SHAPE;
    if (N * (K / 8) > (int64_t(1) << 40)) return W4A16_ERR_SHAPE;
    if (g < 1) return W4A16_ERR_GROUP;
    if (g == K) {
        *G = 1;
        *gshift = 31;
        return W4A16_OK;
    }
    const int sh = log2_exact(g);
    if (sh < 5 || g > K || K % g != 0) return W4A16_ERR_GROUP;
    *G = (int)(K / g);
    *gshift = sh;
    return W4A16_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? W4A16_OK : W4A16_ERR_HIP; }

int validate_linear(const void* X, int dtype, int64_t M, int64_t N, int64_t K, int64_t g,
                    const int32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                    void* Y, LinearArgs* a) {
    if (!X || !qweight || !scales || !Y) return W4A16_ERR_NULL;
    if (dtype != W4A16_F16 && dtype != W4A16_BF16) return W4A16_ERR_DTYPE;
    if (M < 1 || M > kMaxDim) return W4A16_ERR_SHAPE;
    int G = 0, gshift = 0;
    const int st = check_shape_group(N, K, g, &G, &gshift);
    if (st != W4A16_OK) return st;
    if (M * K > (int64_t(1) << 42) || M * N > (int64_t(1) << 42)) return W4A16_ERR_SHAPE;
    if (!aligned(X, 16) || !aligned(qweight, 16) || !aligned(scales, 2) || !aligned(Y, 2) ||
        (zeros && !aligned(zeros, 2)))
        return W4A16_ERR_ALIGN;
    a->X = X;
    a->qw = reinterpret_cast<const uint32_t*>(qweight);
    a->scales = scales;
    a->zeros = zeros;
    a->Y = Y;
    a->dtype = dtype;
    a->M = (int)M;
    a->N = (int)N;
    a->K = (int)K;
    a->G = G;
    a->gshift = gshift;
    a->g = (int)g;
    return W4A16_OK;
}

// M-based dispatch: the weight-streaming GEMV while the dot2 work per weight stays
// within the VALU budget of the HBM stream, the skinny MFMA kernel for small batches,
// the tiled MFMA GEMM once the problem is compute-bound.
// Between 32 and 512 activation rows the tiled GEMM has few tiles and each CU runs one of them
// through the whole K loop, while the skinny kernel splits K over the 8 waves of every block and
// covers the GPU.  Estimated times (microseconds, fitted to MI355X measurements of both kernels
// on the 7B-like prefill shapes for M = 48 .. 512; fp16 picks the faster one at 26 of 27
// measured points): fp16 skinny ~ max(3.9e-3 K, 0.9e-8 M N K), the wide tiled kernel as
// prefill_f16_estimate_us; bf16 skinny ~ max(40, 1.45e-8 M N K), tiled ~ 1.3 (K / 64)
// ceil(tiles / 512) with 128 x 128 tiles, two blocks per CU.
bool skinny_beats_tiled(const LinearArgs& a) {
    const double macs = (double)a.M * a.N * a.K;
    if (a.dtype == W4A16_F16) {
        const double t_tiled = w4a16::prefill_f16_estimate_us(a);
        if (t_tiled > 0.0) return std::max(3.9e-3 * a.K, 0.9e-8 * macs) < t_tiled;
        const long long tiles = ((a.M + 255) / 256) * ((a.N + 255) / 256);
        return std::max(40.0, 1.05e-8 * macs) < 1.45 * (a.K / 64.0) * (double)((tiles + 255) / 256);
    }
    const double t_skinny = std::max(40.0, 1.45e-8 * macs);
    const long long tiles = ((a.M + 127) / 128) * ((a.N + 127) / 128);
    const double t_tiled = 1.3 * (a.K / 64.0) * (double)((tiles + 511) / 512);
    return t_skinny < t_tiled;
}

int choose_path(const LinearArgs& a) {
    // measured on MI355X: the v_dot2 GEMV leads for one row and for two rows of short K
    // (K <= 4096), the MFMA decode kernels (skinny path, 1 <= M <= 16) from there on; one row
    // of K > 24576 streams faster through the MFMA decode kernel's LDS ring (N = 8192:
    // K = 28672 23.9 against 27.2 us, K = 24576 21.8 against 20.8 us)
    const bool long_row = a.M == 1 && a.K > 24576 && w4a16::decode_supports(a);
    if ((a.M == 1 || (a.M == 2 && a.K <= 4096)) && !long_row && w4a16::gemv_supports(a)) return W4A16_PATH_GEMV;
    if (a.M <= 16 && w4a16::decode_supports(a)) return W4A16_PATH_SKINNY;
    if (a.M <= 4 && w4a16::gemv_supports(a)) return W4A16_PATH_GEMV;
    if (a.M <= 32 && w4a16::skinny_supports(a)) return W4A16_PATH_SKINNY;
    if (w4a16::skinny_supports(a) && w4a16::prefill_supports(a) && skinny_beats_tiled(a))
        return W4A16_PATH_SKINNY;
    if (w4a16::prefill_supports(a)) return W4A16_PATH_PREFILL;
    if (w4a16::gemv_supports(a)) return W4A16_PATH_GEMV;
    if (w4a16::skinny_supports(a)) return W4A16_PATH_SKINNY;
    return -1;
}

int run_linear(const LinearArgs& a, int path, hipStream_t s) {
    hipError_t e;
    switch (path) {
        case W4A16_PATH_GEMV:
            if (!w4a16::gemv_supports(a)) return W4A16_ERR_PATH;
            e = w4a16::launch_gemv(a, s);
            break;
        case W4A16_PATH_SKINNY:
            if (!w4a16::skinny_supports(a)) return W4A16_ERR_PATH;
            e = w4a16::launch_skinny(a, s);
            break;
        case W4A16_PATH_PREFILL:
            if (!w4a16::prefill_supports(a)) return W4A16_ERR_PATH;
            e = w4a16::launch_prefill(a, s);
            break;
        default:
            return W4A16_ERR_PATH;
    }
    return hip_status(e);
}

}  // namespace

extern "C" {

int w4a16_abi_version(void) { return W4A16_ABI_VERSION; }

const char* w4a16_strerror(int status) {
    switch (status) {
        case W4A16_OK: return "ok";
        case W4A16_ERR_NULL: return "a required pointer is NULL";
        case W4A16_ERR_SHAPE: return "invalid shape (M, N, K >= 1, K % 32 == 0, size limits)";
        case W4A16_ERR_GROUP:
            return "unsupported group size (g == K, or a power of two >= 32 dividing K)";
        case W4A16_ERR_ALIGN: return "misaligned pointer (X, W, qweight 16 B; others 2 B)";
        case W4A16_ERR_DTYPE: return "unknown activation dtype";
        case W4A16_ERR_SCHEME: return "unknown quantization scheme";
        case W4A16_ERR_HIP: return "HIP runtime error at launch";
        case W4A16_ERR_PATH: return "the requested kernel path does not support this problem";
        case W4A16_ERR_SCRATCH:
            return "the problem needs more workspace than the library's static scratch buffer (64 MiB)";
        default: return "unknown status";
    }
}

int w4a16_quantize_pack(const float* W, int64_t N, int64_t K, int64_t group_size, int scheme,
                        int32_t* qweight, uint16_t* scales, uint16_t* zeros, void* stream) {
    if (!W || !qweight || !scales) return W4A16_ERR_NULL;
    if (scheme != W4A16_ASYM_RTN && scheme != W4A16_SYM_ABSMAX) return W4A16_ERR_SCHEME;
    if (scheme == W4A16_ASYM_RTN && !zeros) return W4A16_ERR_NULL;
    int G = 0, gshift = 0;
    const int st = check_shape_group(N, K, group_size, &G, &gshift);
    if (st != W4A16_OK) return st;
    if (!aligned(W, 16) || !aligned(qweight, 16) || !aligned(scales, 2) ||
        (zeros && !aligned(zeros, 2)))
        return W4A16_ERR_ALIGN;
    const hipError_t e = w4a16::launch_quantize_pack(
        W, (int)N, (int)K, (int)group_size, gshift, scheme, reinterpret_cast<uint32_t*>(qweight),
        scales, zeros, static_cast<hipStream_t>(stream));
    return hip_status(e);
}

int w4a16_dequantize(const int32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                     int64_t N, int64_t K, int64_t group_size, float* out, void* stream) {
    if (!qweight || !scales || !out) return W4A16_ERR_NULL;
    int G = 0, gshift = 0;
    const int st = check_shape_group(N, K, group_size, &G, &gshift);
    if (st != W4A16_OK) return st;
    if (!aligned(qweight, 16) || !aligned(out, 16) || !aligned(scales, 2) ||
        (zeros && !aligned(zeros, 2)))
        return W4A16_ERR_ALIGN;
    const hipError_t e = w4a16::launch_dequantize(reinterpret_cast<const uint32_t*>(qweight),
                                                  scales, zeros, (int)N, (int)K, (int)group_size,
                                                  gshift, out, static_cast<hipStream_t>(stream));
    return hip_status(e);
}

int w4a16_gptq_hessian(const void* X, int dtype, int64_t n_samples, int64_t K, double* H,
                       int accumulate, void* stream) {
    if (!X || !H) return W4A16_ERR_NULL;
    if (dtype != W4A16_F16 && dtype != W4A16_BF16) return W4A16_ERR_DTYPE;
    if (n_samples < 1 || K < 1 || n_samples > kMaxDim || K > kGptqMaxK) return W4A16_ERR_SHAPE;
    if (n_samples * K > (int64_t(1) << 40)) return W4A16_ERR_SHAPE;
    if (!aligned(X, 2) || !aligned(H, 8)) return W4A16_ERR_ALIGN;
    return hip_status(w4a16::launch_gptq_hessian(X, dtype, (int)n_samples, (int)K, H, accumulate != 0,
                                                 static_cast<hipStream_t>(stream)));
}

int w4a16_gptq_factor(double* H, int64_t K, double damp, double* U, void* stream) {
    if (!H || !U) return W4A16_ERR_NULL;
    if (K < 2 || K > kGptqMaxK) return W4A16_ERR_SHAPE;
    if (!(damp >= 0.0) || damp > 1e6) return W4A16_ERR_SHAPE;
    if (!aligned(H, 8) || !aligned(U, 8)) return W4A16_ERR_ALIGN;
    return hip_status(w4a16::launch_gptq_factor(H, (int)K, damp, U, static_cast<hipStream_t>(stream)));
}

int w4a16_gptq_quantize(const float* W, int64_t N, int64_t K, int64_t group_size, int scheme,
                        const double* U, double* work, int32_t* qweight, uint16_t* scales,
                        uint16_t* zeros, void* stream) {
    if (!W || !U || !work || !qweight || !scales) return W4A16_ERR_NULL;
    if (scheme != W4A16_ASYM_RTN && scheme != W4A16_SYM_ABSMAX) return W4A16_ERR_SCHEME;
    if (scheme == W4A16_ASYM_RTN && !zeros) return W4A16_ERR_NULL;
    int G = 0, gshift = 0;
    const int st = check_shape_group(N, K, group_size, &G, &gshift);
    if (st != W4A16_OK) return st;
    if (K > kGptqMaxK || N * K > (int64_t(1) << 34)) return W4A16_ERR_SHAPE;
    if (!aligned(W, 4) || !aligned(U, 8) || !aligned(work, 8) || !aligned(qweight, 4) ||
        !aligned(scales, 2) || (zeros && !aligned(zeros, 2)))
        return W4A16_ERR_ALIGN;
    return hip_status(w4a16::launch_gptq_quantize(W, (int)N, (int)K, (int)group_size, scheme, U, work,
                                                  reinterpret_cast<uint32_t*>(qweight), scales, zeros,
                                                  static_cast<hipStream_t>(stream)));
}

int64_t w4a16_awq_workspace(int64_t N, int64_t K, int64_t n_samples) {
    if (N < 1 || K < 1 || n_samples < 1) return W4A16_ERR_SHAPE;
    return w4a16::awq_workspace_doubles(N, K, n_samples);
}

int w4a16_awq_stats(const void* X, int dtype, int64_t n_samples, int64_t K, float* xmean,
                    void* stream) {
    if (!X || !xmean) return W4A16_ERR_NULL;
    if (dtype != W4A16_F16 && dtype != W4A16_BF16) return W4A16_ERR_DTYPE;
    if (n_samples < 1 || K < 1 || n_samples > kMaxDim || K > kMaxDim) return W4A16_ERR_SHAPE;
    if (n_samples * K > (int64_t(1) << 40)) return W4A16_ERR_SHAPE;
    if (!aligned(X, 2) || !aligned(xmean, 4)) return W4A16_ERR_ALIGN;
    return hip_status(w4a16::launch_awq_stats(X, dtype, (int)n_samples, (int)K, xmean,
                                              static_cast<hipStream_t>(stream)));
}

int w4a16_awq_search(const float* W, int64_t N, int64_t K, const void* X, int dtype,
                     int64_t n_samples, const float* xmean, int64_t group_size, int scheme,
                     double* work, double* losses, int32_t* best, float* s_out, int32_t* qweight,
                     uint16_t* scales, uint16_t* zeros, void* stream) {
    if (!W || !X || !xmean || !work || !losses || !best || !s_out || !qweight || !scales)
        return W4A16_ERR_NULL;
    if (dtype != W4A16_F16 && dtype != W4A16_BF16) return W4A16_ERR_DTYPE;
    if (scheme != W4A16_ASYM_RTN && scheme != W4A16_SYM_ABSMAX) return W4A16_ERR_SCHEME;
    if (scheme == W4A16_ASYM_RTN && !zeros) return W4A16_ERR_NULL;
    int G = 0, gshift = 0;
    const int st = check_shape_group(N, K, group_size, &G, &gshift);
    if (st != W4A16_OK) return st;
    if (n_samples < 1 || n_samples > kMaxDim || N * K > (int64_t(1) << 34) ||
        n_samples * N > (int64_t(1) << 34))
        return W4A16_ERR_SHAPE;
    if (!aligned(W, 4) || !aligned(X, 2) || !aligned(xmean, 4) || !aligned(work, 8) ||
        !aligned(losses, 8) || !aligned(best, 4) || !aligned(s_out, 4) || !aligned(qweight, 4) ||
        !aligned(scales, 2) || (zeros && !aligned(zeros, 2)))
        return W4A16_ERR_ALIGN;
    return hip_status(w4a16::launch_awq_search(
        W, (int)N, (int)K, X, dtype, (int)n_samples, xmean, (int)group_size, scheme, work, losses,
        reinterpret_cast<int*>(best), s_out, reinterpret_cast<uint32_t*>(qweight), scales, zeros,
        static_cast<hipStream_t>(stream)));
}

int w4a16_awq_scale(const void* X, int dtype, int64_t M, int64_t K, const float* s, void* Y,
                    void* stream) {
    if (!X || !s || !Y) return W4A16_ERR_NULL;
    if (dtype != W4A16_F16 && dtype != W4A16_BF16) return W4A16_ERR_DTYPE;
    if (M < 1 || K < 1 || M > kMaxDim || K > kMaxDim || M * K > (int64_t(1) << 42))
        return W4A16_ERR_SHAPE;
    if (!aligned(X, 2) || !aligned(s, 4) || !aligned(Y, 2)) return W4A16_ERR_ALIGN;
    return hip_status(w4a16::launch_awq_scale(X, dtype, M, (int)K, s, Y,
                                              static_cast<hipStream_t>(stream)));
}

int w4a16_w8a8_smooth(const void* X, int dtype, int64_t n_samples, const float* W, int64_t N,
                      int64_t K, int alpha_quarters, float* s, void* stream) {
    if (!X || !W || !s) return W4A16_ERR_NULL;
    if (dtype != W4A16_F16 && dtype != W4A16_BF16) return W4A16_ERR_DTYPE;
    if (n_samples < 1 || N < 1 || K < 1 || n_samples > kMaxDim || N > kMaxDim || K > kMaxDim ||
        n_samples * K > (int64_t(1) << 40) || N * K > (int64_t(1) << 40) || alpha_quarters < 0 ||
        alpha_quarters > 4)
        return W4A16_ERR_SHAPE;
    if (!aligned(X, 2) || !aligned(W, 4) || !aligned(s, 4)) return W4A16_ERR_ALIGN;
    return hip_status(w4a16::launch_w8a8_smooth(X, dtype, (int)n_samples, W, (int)N, (int)K,
                                                alpha_quarters, s, static_cast<hipStream_t>(stream)));
}

int w4a16_w8a8_quantize_weight(const float* W, int64_t N, int64_t K, const float* s,
                               int8_t* qweight, float* wscale, void* stream) {
    if (!W || !s || !qweight || !wscale) return W4A16_ERR_NULL;
    if (N < 1 || K < 1 || N > kMaxDim || K > kMaxDim || N * K > (int64_t(1) << 40))
        return W4A16_ERR_SHAPE;
    if (!aligned(W, 4) || !aligned(s, 4) || !aligned(wscale, 4)) return W4A16_ERR_ALIGN;
    return hip_status(w4a16::launch_w8a8_quant_weight(W, (int)N, (int)K, s, qweight, wscale,
                                                      static_cast<hipStream_t>(stream)));
}

int w4a16_w8a8_quantize_act(const void* X, int dtype, int64_t M, int64_t K, const float* s,
                            int8_t* qx, float* xscale, void* stream) {
    if (!X || !s || !qx || !xscale) return W4A16_ERR_NULL;
    if (dtype != W4A16_F16 && dtype != W4A16_BF16) return W4A16_ERR_DTYPE;
    if (M < 1 || K < 1 || M > kMaxDim || K > kMaxDim || M * K > (int64_t(1) << 40))
        return W4A16_ERR_SHAPE;
    if (!aligned(X, 2) || !aligned(s, 4) || !aligned(xscale, 4)) return W4A16_ERR_ALIGN;
    return hip_status(w4a16::launch_w8a8_quant_act(X, dtype, (int)M, (int)K, s, qx, xscale,
                                                   static_cast<hipStream_t>(stream)));
}

int w4a16_w8a8_linear(const int8_t* qx, const float* xscale, int64_t M, int64_t N, int64_t K,
                      const int8_t* qweight, const float* wscale, void* Y, int dtype,
                      void* stream) {
    if (!qx || !xscale || !qweight || !wscale || !Y) return W4A16_ERR_NULL;
    if (dtype != W4A16_F16 && dtype != W4A16_BF16) return W4A16_ERR_DTYPE;
    if (M < 1 || N < 1 || K < 1 || K % 128 != 0 || M * K >= (int64_t(1) << 31) ||
        N * K >= (int64_t(1) << 31) || M * N > (int64_t(1) << 42) || K > 16777216)
        return W4A16_ERR_SHAPE;
    if (!aligned(qx, 16) || !aligned(qweight, 16) || !aligned(xscale, 4) || !aligned(wscale, 4) ||
        !aligned(Y, 2))
        return W4A16_ERR_ALIGN;
    return hip_status(w4a16::launch_w8a8_linear(qx, xscale, (int)M, (int)N, (int)K, qweight, wscale,
                                                Y, dtype, static_cast<hipStream_t>(stream)));
}

int64_t w4a16_kv_attention_workspace(int64_t Hq, int64_t T, int64_t D) {
    if (Hq < 1 || T < 1 || (D != 64 && D != 128) || Hq > 65535 || T > (int64_t(1) << 24)) return W4A16_ERR_SHAPE;
    return w4a16::kv_attention_workspace_floats(1, Hq, T, D);
}

int64_t w4a16_kv_attention_batch_workspace(int64_t B, int64_t Hq, int64_t Tmax, int64_t D) {
    if (B < 1 || Hq < 1 || Tmax < 1 || (D != 64 && D != 128) || B > 65535 || Hq > 65535 ||
        B * Hq > (int64_t(1) << 24) || Tmax > (int64_t(1) << 24))
        return W4A16_ERR_SHAPE;
    return w4a16::kv_attention_workspace_floats(B, Hq, Tmax, D);
}

int w4a16_kv_quantize(const void* x, int dtype, int64_t H, int64_t T, int64_t D, int bits,
                      void* codes, uint16_t* scales, uint16_t* zeros, void* stream) {
    if (!x || !codes || !scales || (bits == 4 && !zeros)) return W4A16_ERR_NULL;
    if (dtype != W4A16_F16 && dtype != W4A16_BF16) return W4A16_ERR_DTYPE;
    if (bits != 8 && bits != 4) return W4A16_ERR_SCHEME;
    if (H < 1 || T < 1 || (D != 64 && D != 128) || H * T > (int64_t(1) << 33)) return W4A16_ERR_SHAPE;
    if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(scales, 2) || (zeros && !aligned(zeros, 2)))
        return W4A16_ERR_ALIGN;
    return hip_status(w4a16::launch_kv_quantize(x, dtype, H * T, (int)D, bits, codes, scales, zeros,
                                                static_cast<hipStream_t>(stream)));
}

int w4a16_kv_attention_decode(const void* q, int dtype, int64_t Hq, int64_t Hkv, int64_t T,
                              int64_t Tmax, int64_t D, int bits, const void* kcodes,
                              const uint16_t* kscales, const uint16_t* kzeros, const void* vcodes,
                              const uint16_t* vscales, const uint16_t* vzeros, float* work,
                              void* out, void* stream) {
    if (!q || !kcodes || !kscales || !vcodes || !vscales || !work || !out) return W4A16_ERR_NULL;
    if (bits == 4 && (!kzeros || !vzeros)) return W4A16_ERR_NULL;
    if (dtype != W4A16_F16 && dtype != W4A16_BF16) return W4A16_ERR_DTYPE;
    if (bits != 8 && bits != 4) return W4A16_ERR_SCHEME;
    if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Hq > 65535 || T < 1 || T > Tmax ||
        (D != 64 && D != 128) || Hkv * Tmax > (int64_t(1) << 33) || Tmax > (int64_t(1) << 24))
        return W4A16_ERR_SHAPE;
    if (!aligned(q, 16) || !aligned(kcodes, 16) || !aligned(vcodes, 16) || !aligned(kscales, 2) ||
        !aligned(vscales, 2) || (kzeros && !aligned(kzeros, 2)) || (vzeros && !aligned(vzeros, 2)) ||
        !aligned(work, 4) || !aligned(out, 2))
        return W4A16_ERR_ALIGN;
    return hip_status(w4a16::launch_kv_attention(q, dtype, 1, (int)Hq, (int)Hkv, (int)T, nullptr, (int)Tmax,
                                                 (int)D, bits, kcodes, kscales, kzeros, vcodes, vscales,
                                                 vzeros, work, out, static_cast<hipStream_t>(stream)));
}

int w4a16_kv_attention_decode_batch(const void* q, int dtype, int64_t B, int64_t Hq, int64_t Hkv,
                                    const int32_t* lengths, int64_t Tmax, int64_t D, int bits,
                                    const void* kcodes, const uint16_t* kscales, const uint16_t* kzeros,
                                    const void* vcodes, const uint16_t* vscales, const uint16_t* vzeros,
                                    float* work, void* out, void* stream) {
    if (!q || !lengths || !kcodes || !kscales || !vcodes || !vscales || !work || !out) return W4A16_ERR_NULL;
    if (bits == 4 && (!kzeros || !vzeros)) return W4A16_ERR_NULL;
    if (dtype != W4A16_F16 && dtype != W4A16_BF16) return W4A16_ERR_DTYPE;
    if (bits != 8 && bits != 4) return W4A16_ERR_SCHEME;
    if (B < 1 || B > 65535 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Hq > 65535 || B * Hq > (int64_t(1) << 24) ||
        Tmax < 1 || Tmax > (int64_t(1) << 24) || (D != 64 && D != 128) || B * Hkv * Tmax > (int64_t(1) << 33))
        return W4A16_ERR_SHAPE;
    if (!aligned(q, 16) || !aligned(lengths, 4) || !aligned(kcodes, 16) || !aligned(vcodes, 16) ||
        !aligned(kscales, 2) || !aligned(vscales, 2) || (kzeros && !aligned(kzeros, 2)) ||
        (vzeros && !aligned(vzeros, 2)) || !aligned(work, 4) || !aligned(out, 2))
        return W4A16_ERR_ALIGN;
    return hip_status(w4a16::launch_kv_attention(q, dtype, (int)B, (int)Hq, (int)Hkv, (int)Tmax, lengths,
                                                 (int)Tmax, (int)D, bits, kcodes, kscales, kzeros, vcodes,
                                                 vscales, vzeros, work, out, static_cast<hipStream_t>(stream)));
}

int w4a16_select_path(int64_t M, int64_t N, int64_t K, int64_t group_size, int dtype) {
    // Fake, aligned, non-null pointers: only shapes are examined.
    alignas(16) static const unsigned char dummy[16] = {0};
    LinearArgs a;
    const int st = validate_linear(dummy, dtype, M, N, K, group_size,
                                   reinterpret_cast<const int32_t*>(dummy),
                                   reinterpret_cast<const uint16_t*>(dummy), nullptr,
                                   const_cast<unsigned char*>(dummy), &a);
    if (st != W4A16_OK) return st;
    const int p = choose_path(a);
    return p < 0 ? W4A16_ERR_PATH : p;
}

int w4a16_linear_ex(const void* X, int dtype, int64_t M, int64_t N, int64_t K,
                    int64_t group_size, const int32_t* qweight, const uint16_t* scales,
                    const uint16_t* zeros, void* Y, int path, void* stream) {
    LinearArgs a;
    const int st = validate_linear(X, dtype, M, N, K, group_size, qweight, scales, zeros, Y, &a);
    if (st != W4A16_OK) return st;
    if (path == W4A16_PATH_AUTO) {
        path = choose_path(a);
        if (path < 0) return W4A16_ERR_PATH;
    }
    return run_linear(a, path, static_cast<hipStream_t>(stream));
}

int w4a16_linear(const void* X, int dtype, int64_t M, int64_t N, int64_t K, int64_t group_size,
                 const int32_t* qweight, const uint16_t* scales, const uint16_t* zeros, void* Y,
                 void* stream) {
    return w4a16_linear_ex(X, dtype, M, N, K, group_size, qweight, scales, zeros, Y,
                           W4A16_PATH_AUTO, stream);
}

int w4a16_linear_batch(const w4a16_linear_item* items, int count, int dtype, void* stream) {
    if (!items) return W4A16_ERR_NULL;
    if (count < 1 || count > kMaxBatch) return W4A16_ERR_SHAPE;
    std::vector<LinearArgs> args((size_t)count);
    std::vector<int> paths((size_t)count);
    for (int i = 0; i < count; ++i) {
        const w4a16_linear_item& it = items[i];
        const int st = validate_linear(it.X, dtype, it.M, it.N, it.K, it.group_size, it.qweight, it.scales,
                                       it.zeros, it.Y, &args[(size_t)i]);
        if (st != W4A16_OK) return st;
        paths[(size_t)i] = choose_path(args[(size_t)i]);
        if (paths[(size_t)i] < 0) return W4A16_ERR_PATH;
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // Layers that a grouped kernel takes share launches of up to 16 layers, in item order:
    // one-row layers (the streaming GEMV) and layers that run alone on the ring decode
    // kernel (MFMA, up to 16 rows); a group of one and every other layer run as w4a16_linear.
    std::vector<LinearArgs> rows1, ring;
    auto flush = [&](std::vector<LinearArgs>& group, bool gemv) -> int {
        int st = W4A16_OK;
        if (group.size() == 1)
            st = run_linear(group[0], choose_path(group[0]), s);
        else if (!group.empty())
            st = hip_status(gemv ? w4a16::launch_gemv_group(group.data(), (int)group.size(), s)
                                 : w4a16::launch_ring_group(group.data(), (int)group.size(), s));
        group.clear();
        return st;
    };
    for (int i = 0; i < count; ++i) {
        const LinearArgs& a = args[(size_t)i];
        const int p = paths[(size_t)i];
        const bool g1 = w4a16::gemv_group_supports(a);
        // 2-8 rows: the ring group also takes layers whose single call runs the GEMV (two rows of
        // K <= 4096), so a decode step's layers share one launch instead of one launch each
        const bool g2 = !g1 && a.M >= 2 && w4a16::ring_group_supports(a) &&
                        ((p == W4A16_PATH_SKINNY && w4a16::skinny_supports(a)) || p == W4A16_PATH_GEMV);
        if (g1 || g2) {
            std::vector<LinearArgs>& group = g1 ? rows1 : ring;
            group.push_back(a);
            if ((int)group.size() == kGroupLaunch) {
                const int st = flush(group, g1);
                if (st != W4A16_OK) return st;
            }
        } else {
            const int st = run_linear(a, p, s);
            if (st != W4A16_OK) return st;
        }
    }
    const int st = flush(rows1, true);
    if (st != W4A16_OK) return st;
    return flush(ring, false);
}

int64_t w4a16_linear_workspace(int64_t M, int64_t N, int64_t K, int64_t group_size, int dtype) {
    alignas(16) static const unsigned char dummy[16] = {0};
    LinearArgs a;
    const int st = validate_linear(dummy, dtype, M, N, K, group_size, reinterpret_cast<const int32_t*>(dummy),
                                   reinterpret_cast<const uint16_t*>(dummy), nullptr,
                                   const_cast<unsigned char*>(dummy), &a);
    if (st != W4A16_OK) return st;
    return w4a16::prefill_splitk_bytes(a);
}

int w4a16_linear_ws(const void* X, int dtype, int64_t M, int64_t N, int64_t K, int64_t group_size,
                    const int32_t* qweight, const uint16_t* scales, const uint16_t* zeros, void* Y, float* work,
                    int64_t work_bytes, void* stream) {
    LinearArgs a;
    const int st = validate_linear(X, dtype, M, N, K, group_size, qweight, scales, zeros, Y, &a);
    if (st != W4A16_OK) return st;
    if (work && !aligned(work, 16)) return W4A16_ERR_ALIGN;
    const long long need = w4a16::prefill_splitk_bytes(a);
    if (need > 0 && work && work_bytes >= need && w4a16::prefill_supports(a))
        return hip_status(w4a16::launch_prefill_splitk(a, work, static_cast<hipStream_t>(stream)));
    return w4a16_linear_ex(X, dtype, M, N, K, group_size, qweight, scales, zeros, Y, W4A16_PATH_AUTO, stream);
}

int w4a16_linear_ws_noalloc(const void* X, int dtype, int64_t M, int64_t N, int64_t K, int64_t group_size,
                            const int32_t* qweight, const uint16_t* scales, const uint16_t* zeros, void* Y,
                            void* stream) {
    LinearArgs a;
    const int st = validate_linear(X, dtype, M, N, K, group_size, qweight, scales, zeros, Y, &a);
    if (st != W4A16_OK) return st;
    const long long need = w4a16::prefill_splitk_bytes(a);
    if (need > w4a16::kScratchBytes) return W4A16_ERR_SCRATCH;
    if (need > 0 && w4a16::prefill_supports(a)) {
        float* work = nullptr;
        if (w4a16::scratch_device_ptr(&work) != hipSuccess) return W4A16_ERR_HIP;
        return hip_status(w4a16::launch_prefill_splitk(a, work, static_cast<hipStream_t>(stream)));
    }
    return w4a16_linear_ex(X, dtype, M, N, K, group_size, qweight, scales, zeros, Y, W4A16_PATH_AUTO, stream);
}

// ----------------------------------------------------------------- W8A16 (8-bit codes)

int w4a16_w8a16_quantize_pack(const float* W, int64_t N, int64_t K, int64_t group_size, int scheme,
                              int32_t* qweight, uint16_t* scales, uint16_t* zeros, void* stream) {
    if (!W || !qweight || !scales) return W4A16_ERR_NULL;
    if (scheme != W4A16_ASYM_RTN && scheme != W4A16_SYM_ABSMAX) return W4A16_ERR_SCHEME;
    if (scheme == W4A16_ASYM_RTN && !zeros) return W4A16_ERR_NULL;
    int G = 0, gshift = 0;
    const int st = check_shape_group(N, K, group_size, &G, &gshift);
    if (st != W4A16_OK) return st;
    if (!aligned(W, 16) || !aligned(qweight, 16) || !aligned(scales, 2) || (zeros && !aligned(zeros, 2)))
        return W4A16_ERR_ALIGN;
    return hip_status(w4a16::launch_quantize_pack8(W, (int)N, (int)K, (int)group_size, scheme,
                                                   reinterpret_cast<uint32_t*>(qweight), scales, zeros,
                                                   static_cast<hipStream_t>(stream)));
}

namespace {
// W8A16 dispatch: the weight-streaming GEMV for up to 16 activation rows while the packed
// weights are below 2 GiB (measured: 3-10x faster than the tiled GEMM there, whose 256-wide
// tiles leave most CUs idle at small M), else the tiled MFMA GEMM (K and g multiples of 64).
int choose_path8(const LinearArgs& a) {
    if (w4a16::gemv8_supports(a)) return W4A16_PATH_GEMV;
    if (w4a16::prefill8_supports(a)) return W4A16_PATH_PREFILL;
    return -1;
}
}  // namespace

int w4a16_w8a16_select_path(int64_t M, int64_t N, int64_t K, int64_t group_size, int dtype) {
    alignas(16) static const unsigned char dummy[16] = {0};
    LinearArgs a;
    const int st = validate_linear(dummy, dtype, M, N, K, group_size, reinterpret_cast<const int32_t*>(dummy),
                                   reinterpret_cast<const uint16_t*>(dummy), nullptr,
                                   const_cast<unsigned char*>(dummy), &a);
    if (st != W4A16_OK) return st;
    const int p = choose_path8(a);
    return p < 0 ? W4A16_ERR_PATH : p;
}

int w4a16_w8a16_linear_ex(const void* X, int dtype, int64_t M, int64_t N, int64_t K, int64_t group_size,
                          const int32_t* qweight, const uint16_t* scales, const uint16_t* zeros, void* Y,
                          int path, void* stream) {
    LinearArgs a;
    const int st = validate_linear(X, dtype, M, N, K, group_size, qweight, scales, zeros, Y, &a);
    if (st != W4A16_OK) return st;
    if (path == W4A16_PATH_AUTO) {
        path = choose_path8(a);
        if (path < 0) return W4A16_ERR_PATH;
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (path == W4A16_PATH_GEMV) {
        if (!w4a16::gemv8_supports(a)) return W4A16_ERR_PATH;
        return hip_status(w4a16::launch_gemv8(a, s));
    }
    if (path == W4A16_PATH_PREFILL) {
        if (!w4a16::prefill8_supports(a)) return W4A16_ERR_PATH;
        return hip_status(w4a16::launch_prefill8(a, s));
    }
    return W4A16_ERR_PATH;
}

int w4a16_w8a16_linear(const void* X, int dtype, int64_t M, int64_t N, int64_t K, int64_t group_size,
                       const int32_t* qweight, const uint16_t* scales, const uint16_t* zeros, void* Y,
                       void* stream) {
    return w4a16_w8a16_linear_ex(X, dtype, M, N, K, group_size, qweight, scales, zeros, Y, W4A16_PATH_AUTO,
                                 stream);
}

}  // extern "C"
