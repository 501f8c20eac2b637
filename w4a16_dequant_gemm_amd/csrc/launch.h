// Internal launcher interface between the C ABI (api.cpp) and the kernels (*.hip).
// Every launcher assumes its arguments were validated by the caller and only enqueues.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

struct LinearArgs {
    const void* X;          // [M, K] fp16/bf16
    const uint32_t* qw;     // [N, K/8]
    const uint16_t* scales; // [N, G]
    const uint16_t* zeros;  // [N, G] or nullptr (all 8)
    void* Y;                // [M, N]
    int dtype;              // 0 fp16, 1 bf16
    int M, N, K;
    int G;                  // groups per row, K / g
    int gshift;             // log2(g), or 31 when g == K
    int g;                  // group size
};

// Host-side shape support checks of each kernel family (no GPU needed).
bool gemv_supports(const LinearArgs& a);
bool skinny_supports(const LinearArgs& a);
bool decode_supports(const LinearArgs& a);
bool prefill_supports(const LinearArgs& a);

hipError_t launch_quantize_pack(const float* W, int N, int K, int g, int gshift, int scheme,
                                uint32_t* qw, uint16_t* scales, uint16_t* zeros, hipStream_t s);
hipError_t launch_dequantize(const uint32_t* qw, const uint16_t* scales, const uint16_t* zeros,
                             int N, int K, int g, int gshift, float* out, hipStream_t s);
hipError_t launch_gemv(const LinearArgs& a, hipStream_t s);
// grouped launch of independent one-row layers (gemv.hip): at most 16 per launch, one dtype
bool gemv_group_supports(const LinearArgs& a);
hipError_t launch_gemv_group(const LinearArgs* items, int count, hipStream_t s);
hipError_t launch_skinny(const LinearArgs& a, hipStream_t s);
hipError_t launch_decode(const LinearArgs& a, hipStream_t s);
// grouped launch of independent layers that run on the ring decode kernel (decode.hip): at
// most 16 per launch, one dtype; ring_group_supports tells whether a layer alone would run there
bool ring_group_supports(const LinearArgs& a);
hipError_t launch_ring_group(const LinearArgs* items, int count, hipStream_t s);
hipError_t launch_prefill(const LinearArgs& a, hipStream_t s);
// estimated time (us) of the plain fp16 prefill launch on the 4-bit wide kernel, < 0 when another
// kernel would run (host only; for the dispatcher)
double prefill_f16_estimate_us(const LinearArgs& a);
// split-K mode of the fp16 256 x 256 prefill kernel (caller workspace of fp32 partial tiles)
int prefill_splitk_splits(const LinearArgs& a);
long long prefill_splitk_bytes(const LinearArgs& a);
hipError_t launch_prefill_splitk(const LinearArgs& a, float* work, hipStream_t s);
// the library's static per-device scratch (scratch.hip): its size, and its device address on
// the current device (looked up once per device)
constexpr long long kScratchBytes = 64LL << 20;
hipError_t scratch_device_ptr(float** out);
// W8A16 (8-bit codes, four per word): quantize-pack, the decode GEMV and the tiled MFMA GEMM
hipError_t launch_quantize_pack8(const float* W, int N, int K, int g, int scheme, uint32_t* qw,
                                 uint16_t* scales, uint16_t* zeros, hipStream_t s);
bool gemv8_supports(const LinearArgs& a);
hipError_t launch_gemv8(const LinearArgs& a, hipStream_t s);
bool prefill8_supports(const LinearArgs& a);
hipError_t launch_prefill8(const LinearArgs& a, hipStream_t s);

// GPTQ (gptq.hip)
hipError_t launch_gptq_hessian(const void* X, int dtype, int n, int K, double* H, bool accumulate,
                               hipStream_t s);
hipError_t launch_gptq_factor(double* H, int K, double damp, double* U, hipStream_t s);
// W8A8 + SmoothQuant (w8a8.hip)
hipError_t launch_w8a8_smooth(const void* X, int dtype, int n, const float* W, int N, int K, int a,
                              float* s, hipStream_t st);
hipError_t launch_w8a8_quant_weight(const float* W, int N, int K, const float* s, int8_t* q,
                                    float* sw, hipStream_t st);
hipError_t launch_w8a8_quant_act(const void* X, int dtype, int M, int K, const float* s, int8_t* q,
                                 float* sx, hipStream_t st);
hipError_t launch_w8a8_linear(const int8_t* qx, const float* sx, int M, int N, int K,
                              const int8_t* qw, const float* sw, void* Y, int dtype, hipStream_t st);

// KV cache (kv.hip)
long long kv_attention_workspace_floats(long long B, long long Hq, long long T, long long D);
hipError_t launch_kv_quantize(const void* x, int dtype, long long rows, int D, int bits, void* codes,
                              uint16_t* scales, uint16_t* zeros, hipStream_t st);
// B sequences of Hq query heads; lens (device, B entries, clamped into [1, Tmax]) or NULL
// for a common length T.
hipError_t launch_kv_attention(const void* q, int dtype, int B, int Hq, int Hkv, int T, const int* lens,
                               int Tmax, int D, int bits, const void* kc, const uint16_t* ks,
                               const uint16_t* kz, const void* vc, const uint16_t* vs, const uint16_t* vz,
                               float* work, void* out, hipStream_t st);

// AWQ (awq.hip)
long long awq_workspace_doubles(long long N, long long K, long long n);
hipError_t launch_awq_stats(const void* X, int dtype, int n, int K, float* xmean, hipStream_t s);
hipError_t launch_awq_search(const float* W, int N, int K, const void* X, int dtype, int n,
                             const float* xmean, int g, int scheme, double* work, double* losses,
                             int* best, float* s_out, uint32_t* qw, uint16_t* scales,
                             uint16_t* zeros, hipStream_t s);
hipError_t launch_awq_scale(const void* X, int dtype, long long M, int K, const float* s, void* Y,
                            hipStream_t st);
hipError_t launch_gptq_quantize(const float* W, int N, int K, int g, int scheme, const double* U,
                                double* work, uint32_t* qw, uint16_t* scales, uint16_t* zeros,
                                hipStream_t s);

}  // namespace w4a16
