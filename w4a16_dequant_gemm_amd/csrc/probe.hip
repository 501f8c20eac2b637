// Read-rate reference for the benchmark (built as its own library, libw4a16_probe.so; not
// part of the W4A16 C ABI).  One launch reads a contiguous buffer once: each 256-thread
// block covers PER * 4 KB, every thread issues its PER 16-byte loads at once (the same
// one-shot load pattern as the decode kernels), then XORs what it read and writes one word,
// so the launch costs its reads and almost nothing else.  Timed over the bytes of a decode
// step, it gives the rate one launch of that size can reach on this GPU: the ceiling the
// weight-streaming kernels are compared against.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

template <int PER>
__global__ __launch_bounds__(kThreads) void read_probe_kernel(const uint8_t* __restrict__ buf, uint32_t bytes,
                                                              uint32_t* __restrict__ out) {
    // num_records = bytes: loads past the end return zeros without touching memory
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(buf), 0, (int)bytes, 0x00020000);
    const uint32_t base = blockIdx.x * (uint32_t)(PER * kThreads * 16);
    u32x4 v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j)
        v[j] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(base + (threadIdx.x + j * kThreads) * 16), 0, 2);
    uint32_t x = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) x ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    out[blockIdx.x * kThreads + threadIdx.x] = x;
}

}  // namespace

// Blocks (and so 32-bit words of `out`, times 256) one probe launch over `bytes` needs; 0 if
// the size or `per` is not supported (bytes must be below 2 GiB, per one of 4, 8, 16).
extern "C" long long w4a16_probe_blocks(long long bytes, int per) {
    if (bytes <= 0 || bytes >= (1LL << 31) || (per != 4 && per != 8 && per != 16)) return 0;
    const long long span = (long long)per * kThreads * 16;
    return (bytes + span - 1) / span;
}

// One read of `bytes` bytes at device pointer `buf`; `out` (device) holds
// w4a16_probe_blocks(bytes, per) * 256 words.  Returns 0, or -1 for an unsupported size, or the
// HIP error of the launch.
extern "C" int w4a16_probe_read(const void* buf, long long bytes, int per, uint32_t* out, void* stream) {
    const long long blocks = w4a16_probe_blocks(bytes, per);
    if (blocks == 0 || !buf || !out) return -1;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const auto b = static_cast<const uint8_t*>(buf);
    const uint32_t n = (uint32_t)bytes;
    if (per == 4)
        hipLaunchKernelGGL(read_probe_kernel<4>, dim3((unsigned)blocks), dim3(kThreads), 0, st, b, n, out);
    else if (per == 8)
        hipLaunchKernelGGL(read_probe_kernel<8>, dim3((unsigned)blocks), dim3(kThreads), 0, st, b, n, out);
    else
        hipLaunchKernelGGL(read_probe_kernel<16>, dim3((unsigned)blocks), dim3(kThreads), 0, st, b, n, out);
    return (int)hipGetLastError();
}
