/*
 * w4a16.h -- C ABI of the MI355X (gfx950) W4A16 weight-only linear layer.
 *
 * The layer computes Y = X . W_hat^T where W_hat[n][k] = s[n][k/g] * (u[n][k] - z[n][k/g])
 * is rebuilt inside the kernels from 4-bit codes u, a 16-bit scale s and a 16-bit zero
 * point z per group of g consecutive input columns, and is never written back to memory.
 * Sources (five pages on LLM weight quantization):
 *   - affine quantization q = round(x/s) + z and dequantization x ~ s(q - z):
 *     page "量化实战深入（GPTQ / AWQ / SmoothQuant / KV 量化）", section 二 (量化的数学本质);
 *     page "推理优化中“用精度换性能“的核心技术：量化", section 2.3 (核心公式);
 *   - asymmetric s = (max-min)/(2^b-1), z = round(-min/s) and symmetric absmax
 *     s = max|x|/(2^(b-1)-1), z = 0: page 4, section 3.3; page 3, section 二;
 *   - INT4 code ranges [0,15] / [-8,7]: page 4, section 2.2;
 *   - group-wise granularity, one 16-bit scale and optional 16-bit zero point per 128
 *     weights (4.25 bits per weight): page 4, section 3.4;
 *   - weight-only quantization keeps activations in FP16/BF16 and dequantizes the INT4
 *     weights for the matrix product: page 4, section 3.2; the dequantization belongs
 *     inside the GEMM, unpacking and scaling in registers or shared memory while the
 *     INT4 data is read: page "大模型推理中 Weight-only、W8A8 和 FP8 量化有什么区别？如何选型？",
 *     section 二, and page "LLM 量化中 W4A16 表示什么，它在权重位宽和激活精度上有什么取舍？",
 *     section 性能取决于 kernel.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library never
 *     allocates device memory, never frees, never synchronizes the device and keeps no
 *     state between calls (thread-safe, re-entrant).  Work is enqueued on `stream`
 *     (a hipStream_t passed as void*; NULL means the default stream) and runs
 *     asynchronously: the caller keeps every buffer alive until that work completes.
 *   - Row-major layouts.  W, X, Y, qweight, scales, zeros are dense (no strides).
 *   - Packed weights: qweight is int32 [N, K/8]; element k of row n is the 4-bit code in
 *     bits 4*(k%8) .. 4*(k%8)+3 of word qweight[n][k/8] (little-endian nibbles).
 *   - scales and zeros are IEEE fp16 bit patterns (uint16) of shape [N, K/g].  Symmetric
 *     weights store codes offset-binary (u = q + 8) with zero point 8; `zeros == NULL` in
 *     w4a16_linear means "all zero points are 8".
 *   - Return value: W4A16_OK (0) or a negative w4a16_status.  Argument errors are detected
 *     on the host before anything is enqueued; W4A16_ERR_HIP reports a failed launch.
 *   - Inputs must be finite; results for NaN/Inf inputs are unspecified.  X and Y must
 *     not overlap qweight/scales/zeros or each other.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A16_ABI_VERSION 1

typedef enum {
    W4A16_OK = 0,
    W4A16_ERR_NULL = -1,    /* a required pointer is NULL                          */
    W4A16_ERR_SHAPE = -2,   /* M, N or K < 1, K % 32 != 0, or a size limit exceeded */
    W4A16_ERR_GROUP = -3,   /* unsupported group size (see below)                  */
    W4A16_ERR_ALIGN = -4,   /* a pointer is not aligned as required                 */
    W4A16_ERR_DTYPE = -5,   /* unknown activation dtype                             */
    W4A16_ERR_SCHEME = -6,  /* unknown quantization scheme                          */
    W4A16_ERR_HIP = -7,     /* the HIP runtime reported an error at launch          */
    W4A16_ERR_PATH = -8,    /* a forced kernel path cannot run this problem         */
    W4A16_ERR_SCRATCH = -9  /* the static scratch buffer is too small (see below)    */
} w4a16_status;

typedef enum { W4A16_F16 = 0, W4A16_BF16 = 1 } w4a16_dtype;

typedef enum {
    W4A16_ASYM_RTN = 0,     /* s = (max-min)/15, z = round(-min/s), codes [0,15]    */
    W4A16_SYM_ABSMAX = 1    /* s = max|x|/7, signed codes [-8,7] stored as q+8      */
} w4a16_scheme;

typedef enum {
    W4A16_PATH_AUTO = 0,    /* dispatcher chooses from (M, N, K, g)                 */
    W4A16_PATH_GEMV = 1,    /* weight-streaming dot2 kernel, any supported g, M<=8  */
    W4A16_PATH_SKINNY = 2,  /* K-split MFMA kernel, M <= 512, g % 128 == 0         */
    W4A16_PATH_PREFILL = 3  /* LDS-tiled MFMA GEMM; bf16 needs g % 64 == 0, K % 64 == 0 */
} w4a16_path;

/*
 * Group-size rule for every entry point: g == K, or g is a power of two with
 * 32 <= g <= K and K % g == 0.  Size limits: 1 <= M, N, K <= 2^31 - 1 and K % 32 == 0.
 */

/*
 * w4a16_quantize_pack -- group-wise round-to-nearest INT4 quantization and packing.
 *   W        [N, K] fp32, device, 16-byte aligned.
 *   scheme   W4A16_ASYM_RTN or W4A16_SYM_ABSMAX.
 *   qweight  out [N, K/8] int32, device, 16-byte aligned.
 *   scales   out [N, K/g] fp16 bits, device, 2-byte aligned.
 *   zeros    out [N, K/g] fp16 bits, device, 2-byte aligned; may be NULL for the symmetric
 *            scheme (then nothing is written; pass NULL zeros to w4a16_linear).
 * Arithmetic per group (IEEE fp32, round-to-nearest-even, this order):
 *   asymmetric: s32 = (max - min) / 15; s = fp16(s32), or 1.0 if that is 0;
 *               z = rint(-min / s) + 0.0; q = clamp(rint(x / s) + z, 0, 15);
 *   symmetric:  s32 = max|x| / 7; s as above; q = clamp(rint(x / s), -8, 7) + 8; z = 8.
 * The result is bit-identical to that arithmetic.  Preconditions: |z| <= 2048 and a
 * finite fp16 scale (otherwise the stored values are unspecified).
 */
int w4a16_quantize_pack(const float* W, int64_t N, int64_t K, int64_t group_size, int scheme,
                        int32_t* qweight, uint16_t* scales, uint16_t* zeros, void* stream);

/*
 * w4a16_linear -- Y[M, N] = X[M, K] . W_hat[N, K]^T with W_hat rebuilt from
 * (qweight, scales, zeros) inside the kernel; fp32 accumulation; Y is rounded once to
 * the activation dtype (round-to-nearest-even).
 *   X        [M, K] fp16 or bf16 (dtype), device, 16-byte aligned.
 *   qweight  [N, K/8] int32, device, 16-byte aligned.
 *   scales   [N, K/g] fp16 bits, device, 2-byte aligned.
 *   zeros    [N, K/g] fp16 bits, device, 2-byte aligned, or NULL (all zero points 8).
 *            Zero points must be integers with |z| <= 2048, the range w4a16_quantize_pack
 *            emits (z is in [0, 15] for every group whose range contains 0; larger |z|
 *            arise for a group far narrower than its distance from 0).  Every kernel path
 *            takes the whole range exactly: the decode kernels and the bf16 GEMM apply z to
 *            fp32 partial sums; the fp16 GEMM rounds s * (u - z), exact in fp32, once to fp16
 *            per weight.
 *   Y        out [M, N], same dtype as X, device, 2-byte aligned.
 * Other zero points give unspecified output (never an out-of-bounds access).
 */
int w4a16_linear(const void* X, int dtype, int64_t M, int64_t N, int64_t K, int64_t group_size,
                 const int32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                 void* Y, void* stream);

/*
 * w4a16_linear_ex -- w4a16_linear with an explicit kernel path (w4a16_path).  A forced
 * path that does not support the problem returns W4A16_ERR_PATH without launching.
 * Intended for testing every kernel at every size it supports.
 */
int w4a16_linear_ex(const void* X, int dtype, int64_t M, int64_t N, int64_t K,
                    int64_t group_size, const int32_t* qweight, const uint16_t* scales,
                    const uint16_t* zeros, void* Y, int path, void* stream);

/*
 * w4a16_linear_batch -- several independent linear layers in one call, for a decode step that
 * runs many layers on the same token (for example the q, k and v projections, or the experts
 * of a mixture, or any set of layers whose inputs are ready).  Each item is a w4a16_linear
 * problem with the call's activation dtype:
 *   X        [M, K] fp16 or bf16, device, 16-byte aligned;
 *   M, N, K, group_size, qweight, scales, zeros, Y  as for w4a16_linear.
 * Every item is validated before anything is enqueued; the first invalid item's status is
 * returned and nothing runs.  Items with M = 1 that the weight-streaming GEMV takes
 * (K <= 12288, packed weights < 2 GiB) share launches of up to 16 layers, in item order: one
 * grid streams all of their weights, so the fixed cost of a launch (dispatch, ramp-up and
 * drain, about as long as streaming a 7B-sized layer at decode) is paid once per group.
 * Items with 2 <= M <= 8 that w4a16_linear runs on its small-batch path or on the GEMV (two
 * rows of K <= 4096), with N and K at most 12288 (K % 256 == 0, group_size % 128 == 0),
 * likewise share launches of up to 16 layers of the MFMA ring decode kernel, one 16-row tile
 * per block, so the layers' blocks overlap (a group of one runs as w4a16_linear).  The
 * other items run as w4a16_linear, in item order.  Grouped outputs meet w4a16_linear's
 * accuracy contract; they are computed with the arithmetic of the kernel the group runs, in
 * the same order, so where w4a16_linear takes that kernel for the layer (the weight-streaming
 * GEMV for every 7B-shaped layer at M = 1 and g = 128; the ring kernel from M = 5) the two
 * results are identical bit for bit.  Items run concurrently: no item's Y may overlap another
 * item's inputs or output.
 *   items    host array of `count` descriptors (read during the call only); 1 <= count <= 65536.
 */
typedef struct {
    const void* X;
    int64_t M, N, K, group_size;
    const int32_t* qweight;
    const uint16_t* scales;
    const uint16_t* zeros;
    void* Y;
} w4a16_linear_item;

int w4a16_linear_batch(const w4a16_linear_item* items, int count, int dtype, void* stream);

/*
 * w4a16_select_path -- the path W4A16_PATH_AUTO would take for this problem (host only,
 * no GPU needed), or a negative status if the arguments are invalid.
 */
int w4a16_select_path(int64_t M, int64_t N, int64_t K, int64_t group_size, int dtype);

/*
 * w4a16_dequantize -- W_hat[N, K] = s * (u - z) as fp32 (exact), for layout checks.
 *   out [N, K] fp32, device, 16-byte aligned; zeros may be NULL (all 8).
 */
int w4a16_dequantize(const int32_t* qweight, const uint16_t* scales, const uint16_t* zeros,
                     int64_t N, int64_t K, int64_t group_size, float* out, void* stream);

/*
 * GPTQ: column-by-column INT4 quantization with second-order error compensation, writing
 * the same packed format as w4a16_quantize_pack.  Page "推理优化中“用精度换性能“的核心技术：
 * 量化", section 四 (4.2 algorithm: H = 2 X^T X, columns quantized in order, every later
 * column j corrected by -dw * Hinv[i, j] / Hinv[i, i]; 4.4 natural column order, Cholesky
 * factor, group_size); page "量化实战深入（GPTQ / AWQ / SmoothQuant / KV 量化）", 4.1.
 * Hinv is the inverse Hessian of the columns not yet quantized; with H^-1 = U^T U (U upper
 * triangular) the correction ratio is U[i, j] / U[i, i].  All compensation arithmetic is
 * fp64; codes, scales and zero points follow the RTN rules of w4a16_quantize_pack applied,
 * at each group's first column, to the group's current (compensated) weights rounded to
 * fp32.  Calls are asynchronous on `stream` like every entry point; the caller owns all
 * buffers.  Typical use: hessian (once, or once per calibration batch with accumulate = 1),
 * factor, quantize.
 */

/*
 * w4a16_gptq_hessian -- H (=, or += when accumulate != 0) 2 X^T X.
 *   X  [n_samples, K] fp16 or bf16 (dtype) calibration activations of the layer, device,
 *      2-byte aligned.
 *   H  [K, K] fp64, device, 8-byte aligned.  Only the lower triangle (i >= j) is defined
 *      on return; the strictly upper part is unspecified.  K <= 46340.
 */
int w4a16_gptq_hessian(const void* X, int dtype, int64_t n_samples, int64_t K, double* H,
                       int accumulate, void* stream);

/*
 * w4a16_gptq_factor -- U = upper Cholesky factor of (H + lambda I)^-1, H^-1 = U^T U, with
 * lambda = damp * mean(diag H) (damp = 0 leaves H as is; 0.01 is customary when the
 * calibration set is small).
 *   H  [K, K] fp64, device: reads the lower triangle; DESTROYED (used as workspace).
 *   U  [K, K] fp64 out, device: upper triangle, zeros below the diagonal.
 * If H + lambda I is not numerically positive definite U contains NaN.
 */
int w4a16_gptq_factor(double* H, int64_t K, double damp, double* U, void* stream);

/*
 * w4a16_gptq_quantize -- GPTQ of W [N, K] fp32 (device, 4-byte aligned) with the factor U
 * from w4a16_gptq_factor.  group_size and scheme as in w4a16_quantize_pack.
 *   work     device fp64 workspace of N * K + 64 * N elements (8-byte aligned).
 *   qweight  out [N, K/8] int32; scales, zeros out [N, K/g] fp16 bits (zeros may be NULL
 *            for the symmetric scheme, else all 8.0).
 * Limits: N * K <= 2^34, K <= 46340.
 */
int w4a16_gptq_quantize(const float* W, int64_t N, int64_t K, int64_t group_size, int scheme,
                        const double* U, double* work, int32_t* qweight, uint16_t* scales,
                        uint16_t* zeros, void* stream);

/*
 * AWQ: activation-aware per-input-channel scaling before group-wise RTN.  Page
 * "推理优化中“用精度换性能“的核心技术：量化", section 五 (5.1 channel importance from the mean
 * activation magnitude on calibration data; 5.2 the exact rescaling
 * W x = (W diag(1/s)) (diag(s) x), the scale chosen by a grid search on the quantized
 * layer's output error; 5.3 plain per-group quantization afterwards); page "量化实战深入
 * （GPTQ / AWQ / SmoothQuant / KV 量化）", 4.2.  Candidates are s = r^(a/4), a = -4 .. 4, with
 * r = xc / sqrt(max xc * min xc), xc = max(xmean, 1e-6 * max xmean); a = 0 is plain RTN.
 * The quantizer sees the fp32 quotient W / s; at inference the activations must be
 * multiplied by s (w4a16_awq_scale, or folded into the preceding operator).
 */

/* Number of fp64 elements of the w4a16_awq_search workspace (host only), or a negative
 * status. */
int64_t w4a16_awq_workspace(int64_t N, int64_t K, int64_t n_samples);

/*
 * w4a16_awq_stats -- xmean[k] = mean over the n_samples rows of |X[t][k]| (fp64 sum, fp32
 * result).  X [n_samples, K] fp16/bf16 device (2-byte aligned); xmean [K] fp32 device.
 */
int w4a16_awq_stats(const void* X, int dtype, int64_t n_samples, int64_t K, float* xmean,
                    void* stream);

/*
 * w4a16_awq_search -- for each of the nine candidates quantize W / s with the RTN rules of
 * w4a16_quantize_pack and measure ||X W^T - (X diag(s)) (W_hat')^T||_F^2 in fp64 on the
 * calibration rows X [n_samples, K]; keep the first minimum.
 *   W        [N, K] fp32 device (4-byte aligned).
 *   xmean    [K] fp32 device, from w4a16_awq_stats (or any positive channel statistic).
 *   work     fp64 device workspace of w4a16_awq_workspace(N, K, n_samples) elements.
 *   losses   out [9] fp64 device: the error of each candidate, a = -4 .. 4.
 *   best     out [1] int32 device: index into losses of the chosen candidate.
 *   s_out    out [K] fp32 device: the chosen scales s.
 *   qweight, scales, zeros: out, the packed quantization of W / s (zeros may be NULL for
 *            the symmetric scheme).
 * Limits: N * K <= 2^34, n_samples * N <= 2^34.
 */
int w4a16_awq_search(const float* W, int64_t N, int64_t K, const void* X, int dtype,
                     int64_t n_samples, const float* xmean, int64_t group_size, int scheme,
                     double* work, double* losses, int32_t* best, float* s_out, int32_t* qweight,
                     uint16_t* scales, uint16_t* zeros, void* stream);

/*
 * w4a16_awq_scale -- Y[m][k] = X[m][k] * s[k] rounded once to the dtype of X (the exact
 * product, round-to-nearest-even).  X, Y [M, K] fp16/bf16 device (2-byte aligned, may be the
 * same buffer); s [K] fp32 device.
 */
int w4a16_awq_scale(const void* X, int dtype, int64_t M, int64_t K, const float* s, void* Y,
                    void* stream);

/*
 * W8A8 with SmoothQuant: both operands in INT8 for the integer matrix units, the activation
 * outlier channels migrated into the weights.  Page "大模型推理中 Weight-only、W8A8 和 FP8 量化有
 * 什么区别？如何选型？", section 三 (Y = (X/s)(sW), INT8 matrix units); page "推理优化中“用精度换
 * 性能“的核心技术：量化", 6.2 (s_j = max|X_j|^alpha / max|W_j|^(1-alpha), alpha = 0.5), 3.3-3.4
 * (symmetric absmax scales, per channel for weights, per token for activations); page
 * "Quantization & Acceleration: 解释 W8A8 与 W4A16 的差异与取舍" (per-token dynamic activation
 * scales).  All fp32 arithmetic follows one fixed order, so codes, scales and outputs are
 * bit-reproducible: alpha = alpha_quarters / 4 with powers formed from square roots and
 * products; w * s_j and x / s_j rounded once; scale = amax / 127 (1.0 if amax is 0); code =
 * clamp(rint(v / scale), -128, 127); Y = out(fp32(fp32(acc) * xscale[m]) * wscale[n]) from
 * the exact int32 sum acc.  Scales are fp32.
 */

/*
 * w4a16_w8a8_smooth -- s[j] = max_t |X[t][j]|^alpha / max_n |W[n][j]|^(1-alpha) (1.0 for a
 * channel whose activation or weight maximum is 0).  X [n_samples, K] fp16/bf16 calibration
 * activations; W [N, K] fp32; s [K] fp32 out; all device.  alpha_quarters in 0..4.
 */
int w4a16_w8a8_smooth(const void* X, int dtype, int64_t n_samples, const float* W, int64_t N,
                      int64_t K, int alpha_quarters, float* s, void* stream);

/*
 * w4a16_w8a8_quantize_weight -- qweight[n][k] = INT8 of W[n][k] * s[k] with one scale per
 * output row n (wscale [N] fp32 out).  W [N, K] fp32, qweight [N, K] int8, device.
 */
int w4a16_w8a8_quantize_weight(const float* W, int64_t N, int64_t K, const float* s,
                               int8_t* qweight, float* wscale, void* stream);

/*
 * w4a16_w8a8_quantize_act -- per-token dynamic INT8 of X[m][k] / s[k] (xscale [M] fp32 out).
 * X [M, K] fp16/bf16, qx [M, K] int8, device.
 */
int w4a16_w8a8_quantize_act(const void* X, int dtype, int64_t M, int64_t K, const float* s,
                            int8_t* qx, float* xscale, void* stream);

/*
 * w4a16_w8a8_linear -- Y[m][n] = out((sum_k qx[m][k] qweight[n][k]) * xscale[m] * wscale[n])
 * on the INT8 matrix cores.  qx [M, K] and qweight [N, K] int8 (16-byte aligned), K % 128 == 0,
 * M * K and N * K < 2^31; Y [M, N] in dtype (fp16/bf16), 2-byte aligned.
 */
int w4a16_w8a8_linear(const int8_t* qx, const float* xscale, int64_t M, int64_t N, int64_t K,
                      const int8_t* qweight, const float* wscale, void* Y, int dtype,
                      void* stream);

/*
 * KV-cache quantization and the decode attention that reads the quantized cache.  Page
 * "量化实战深入（GPTQ / AWQ / SmoothQuant / KV 量化）", 六 KV Cache 量化 (KV8 / KV4, keys and
 * values quantized separately, per token); page "Quantization & Acceleration: 解释 W8A8 与 W4A16
 * 的差异与取舍", 深度剖析 ③ (W4A16 + KV INT8).  One scale (KV4: and zero point) per (head,
 * token) row of D values.  KV8: s = fp16(max|x| / 127) (1.0 if 0), int8 codes
 * clamp(rint(x / s), -127, 127); KV4: the asymmetric RTN of w4a16_quantize_pack with g = D,
 * nibbles packed as in qweight.  Cache layout [H, Tmax, D] (codes: int8, or int32 words of 8
 * nibbles), scales / zeros [H, Tmax] fp16.  D is 64 or 128.
 */

/*
 * w4a16_kv_quantize -- quantize x [H, T, D] (fp16/bf16, 16-byte aligned) into codes
 * (int8 [H, T, D] or int32 [H, T, D/8], 8-byte aligned), scales and, for bits == 4, zeros
 * ([H, T] fp16).  Rows are independent: quantizing new tokens of a cache is a call on their
 * rows (with the cache's row stride equal to T of that call's layout).
 */
int w4a16_kv_quantize(const void* x, int dtype, int64_t H, int64_t T, int64_t D, int bits,
                      void* codes, uint16_t* scales, uint16_t* zeros, void* stream);

/* fp32 elements of the w4a16_kv_attention_decode workspace (host only), or a negative status. */
int64_t w4a16_kv_attention_workspace(int64_t Hq, int64_t T, int64_t D);

/*
 * w4a16_kv_attention_decode -- out[h] = softmax(q[h] . K_t / sqrt(D)) V over the first T of
 * Tmax cached tokens of kv head h / (Hq / Hkv) (grouped-query attention when Hq > Hkv).
 *   q    [Hq, D] fp16/bf16, 16-byte aligned; out [Hq, D] same dtype.
 *   kcodes, vcodes / kscales, vscales / kzeros, vzeros: the caches of w4a16_kv_quantize with
 *        H = Hkv and T = Tmax <= 2^24 (zeros only for bits == 4; 16-byte aligned codes).
 *   work w4a16_kv_attention_workspace(Hq, T, D) fp32 elements (scratch, contents undefined
 *        after the call; calls that overlap on one work buffer race).
 * Scores and softmax in fp32 (max-subtracted, base-2 exponentials with q prescaled by
 * log2(e) / sqrt(D)), each split of tokens reduced with an online softmax, the splits merged
 * by a second launch; the output is rounded once.  The cache is read once per group of up to
 * 4 (KV8) or 2 (KV4) query heads that share a kv head.
 */
int w4a16_kv_attention_decode(const void* q, int dtype, int64_t Hq, int64_t Hkv, int64_t T,
                              int64_t Tmax, int64_t D, int bits, const void* kcodes,
                              const uint16_t* kscales, const uint16_t* kzeros, const void* vcodes,
                              const uint16_t* vscales, const uint16_t* vzeros, float* work,
                              void* out, void* stream);

/* fp32 elements of the w4a16_kv_attention_decode_batch workspace (host only), or a negative
 * status. */
int64_t w4a16_kv_attention_batch_workspace(int64_t B, int64_t Hq, int64_t Tmax, int64_t D);

/*
 * w4a16_kv_attention_decode_batch -- decode attention for a batch of B sequences, each over its
 * own quantized cache, in one pair of launches: out[b][h] = softmax(q[b][h] . K_bt / sqrt(D)) V_b
 * over the first lengths[b] tokens of sequence b, kv head h / (Hq / Hkv).  The serving case the
 * cache quantization is for: more concurrent sequences in the same memory (page
 * "量化实战深入（GPTQ / AWQ / SmoothQuant / KV 量化）", 六 KV Cache 量化).
 *   q        [B, Hq, D] fp16/bf16, 16-byte aligned; out [B, Hq, D] same dtype.
 *   lengths  device int32 [B]; each value is clamped into [1, Tmax] on the device.
 *   caches   w4a16_kv_quantize output with H = B * Hkv and T = Tmax ([B, Hkv, Tmax, ...]).
 *   work     w4a16_kv_attention_batch_workspace(B, Hq, Tmax, D) fp32 elements (scratch).
 * Same arithmetic as w4a16_kv_attention_decode; B <= 65535, Tmax <= 2^24.
 */
int w4a16_kv_attention_decode_batch(const void* q, int dtype, int64_t B, int64_t Hq, int64_t Hkv,
                                    const int32_t* lengths, int64_t Tmax, int64_t D, int bits,
                                    const void* kcodes, const uint16_t* kscales, const uint16_t* kzeros,
                                    const void* vcodes, const uint16_t* vscales, const uint16_t* vzeros,
                                    float* work, void* out, void* stream);

/*
 * w4a16_linear_workspace -- bytes of fp32 workspace that w4a16_linear_ws can use for this
 * problem (0: it would not split K and behaves as w4a16_linear); a negative status for invalid
 * arguments.  Host only.
 */
int64_t w4a16_linear_workspace(int64_t M, int64_t N, int64_t K, int64_t group_size, int dtype);

/*
 * w4a16_linear_ws -- w4a16_linear with a caller workspace for the prefill regime's tile-starved
 * shapes (fp16, M > 32, K % 128 == 0, fewer than 128 tiles of 256 x 256): the 256 x 256 kernel
 * then splits K over the otherwise idle CUs, writes fp32 partial tiles to `work` and a second
 * kernel sums them in split order and rounds once, so the result is deterministic (the same
 * dequantized weights and products as w4a16_linear, summed in a different order).  The compute
 * regime the pages assign to prefill (page "Quantization & Acceleration: 解释 W8A8 与 W4A16 的
 * 差异与取舍", prefill compute-bound).
 *   work        device fp32, 16-byte aligned, at least w4a16_linear_workspace(...) bytes
 *               (scratch, overwritten); NULL or smaller: the call is w4a16_linear.
 *   work_bytes  its size in bytes.  Other arguments as for w4a16_linear.
 */
int w4a16_linear_ws(const void* X, int dtype, int64_t M, int64_t N, int64_t K, int64_t group_size,
                    const int32_t* qweight, const uint16_t* scales, const uint16_t* zeros, void* Y, float* work,
                    int64_t work_bytes, void* stream);

/*
 * w4a16_linear_ws_noalloc -- w4a16_linear_ws with the library's own static scratch buffer as
 * the workspace, so the call allocates nothing and needs no caller memory beyond X, the weights
 * and Y.  For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).
 *   The buffer holds 64 MiB per GPU: a file-scope device array, so every GPU the library runs
 *   on holds its own copy until the process ends.  Its address on the current device is looked
 *   up on the first call on that device (no allocation); the stream must belong to the current
 *   device.  The split never needs more than 64 MiB (at most 256 partial fp32 tiles of
 *   256 x 256); a problem that would (w4a16_linear_workspace(...) > 64 MiB) returns
 *   W4A16_ERR_SCRATCH without launching.  Problems that do not split K run as w4a16_linear.
 *   Results are bit-identical to w4a16_linear_ws with a large enough workspace.
 *   Every call on one GPU shares that GPU's buffer and leaves its partial tiles in it: calls
 *   that overlap on one GPU (several streams, several host threads) race and give undefined
 *   results; serialize them.  Other arguments and errors as for w4a16_linear.
 */
int w4a16_linear_ws_noalloc(const void* X, int dtype, int64_t M, int64_t N, int64_t K, int64_t group_size,
                            const int32_t* qweight, const uint16_t* scales, const uint16_t* zeros, void* Y,
                            void* stream);

/* ------------------------------------------------------------------------------------
 * W8A16: the same weight-only layer with 8-bit codes, four per 32-bit word (byte k % 4 of
 * word k / 4 is element k) and the same fp16 scale and zero point per group (page
 * "大模型推理中 Weight-only、W8A8 和 FP8 量化有什么区别？如何选型？", 二, INT8 / INT4 weight-only
 * with 16-bit activations; page "推理优化中“用精度换性能“的核心技术：量化", 3.3, the 8-bit
 * asymmetric divisor 255).  Shapes, group sizes, alignment and status codes follow the 4-bit
 * calls; qweight is [N, K/4] int32.
 */

/*
 * w4a16_w8a16_quantize_pack -- group-wise round-to-nearest INT8 quantization and packing.
 *   W        [N, K] fp32, device, 16-byte aligned.
 *   qweight  out [N, K/4] int32, device, 16-byte aligned.
 *   scales   out [N, K/g] fp16 bits; zeros out [N, K/g] fp16 bits, or NULL for the symmetric
 *            scheme (the implicit zero point is then 128).
 * Arithmetic per group (IEEE fp32, round-to-nearest-even, this order):
 *   asymmetric: s32 = (max - min) / 255; s = fp16(s32), or 1.0 if that is 0;
 *               z = rint(-min / s) + 0.0; u = clamp(rint(x / s) + z, 0, 255);
 *   symmetric:  s32 = max|x| / 127; s as above; u = clamp(rint(x / s), -128, 127) + 128; z = 128.
 * Bit-identical to that arithmetic; preconditions as for w4a16_quantize_pack.
 */
int w4a16_w8a16_quantize_pack(const float* W, int64_t N, int64_t K, int64_t group_size, int scheme,
                              int32_t* qweight, uint16_t* scales, uint16_t* zeros, void* stream);

/*
 * w4a16_w8a16_linear -- Y[M, N] = X[M, K] . W_hat[N, K]^T, W_hat[n, k] = s (u - z) from the
 * 8-bit codes, dequantized inside the kernel (the GEMV and the bf16 GEMM multiply the exact
 * codes and apply the group's s and z to fp32 partial sums; the fp16 GEMM rounds s * (u - z),
 * exact in fp32, once to fp16 per weight);
 * fp32 accumulation, Y rounded once to the activation dtype.  Arguments as for w4a16_linear
 * with qweight [N, K/4]; zeros NULL means all zero points 128; any integer zero point
 * |z| <= 2048 (the range w4a16_w8a16_quantize_pack emits).  Kernels: a weight-streaming GEMV
 * for M <= 16 (when N * K < 2^31), else the tiled MFMA GEMM, which needs K and g to be
 * multiples of 64 (W4A16_ERR_PATH otherwise).
 */
int w4a16_w8a16_linear(const void* X, int dtype, int64_t M, int64_t N, int64_t K, int64_t group_size,
                       const int32_t* qweight, const uint16_t* scales, const uint16_t* zeros, void* Y,
                       void* stream);

/* w4a16_w8a16_linear with an explicit kernel: W4A16_PATH_AUTO, W4A16_PATH_GEMV or
 * W4A16_PATH_PREFILL (W4A16_ERR_PATH when that kernel cannot take the problem). */
int w4a16_w8a16_linear_ex(const void* X, int dtype, int64_t M, int64_t N, int64_t K, int64_t group_size,
                          const int32_t* qweight, const uint16_t* scales, const uint16_t* zeros, void* Y,
                          int path, void* stream);

/* The kernel w4a16_w8a16_linear would take (host only; a negative status for invalid shapes). */
int w4a16_w8a16_select_path(int64_t M, int64_t N, int64_t K, int64_t group_size, int dtype);

/* Human-readable text for a status code (static storage). */
const char* w4a16_strerror(int status);

/* W4A16_ABI_VERSION of the built library. */
int w4a16_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
