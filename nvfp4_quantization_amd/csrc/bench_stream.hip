// Streaming kernel with the memory traffic of a 1x16 quantization and none of its arithmetic: the practical
// bandwidth ceiling that the quantizers are compared against.  Built into its own library (libnvfp4_bench.so);
// it is not part of the NVFP4 C ABI.
//
// Per 16-element block: 32 bytes read (the bf16 values), 8 bytes written (where the codes would go) and 1 byte
// written (where the scale would go), i.e. 2 + 0.5 + 1/16 bytes per element, the same mix as the quantizers.
// The written values are xor folds of what was read, so the loads cannot be elided.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 1;  // blocks per lane (1, 2, 4 and 8 measured; 1 was fastest at 8192 x 4096)

typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));

__global__ void __launch_bounds__(kThreads)
k_stream_blocks(const uint4* __restrict__ x, uint64_t nblocks, u32x2v* __restrict__ codes,
                uint8_t* __restrict__ scales) {
    uint4 a[kUnroll], b[kUnroll];
    const uint64_t base = (uint64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const uint64_t n = base + (uint64_t)u * kThreads;
        if (n < nblocks) {
            a[u] = x[2 * n];
            b[u] = x[2 * n + 1];
        }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const uint64_t n = base + (uint64_t)u * kThreads;
        if (n < nblocks) {
            const uint32_t lo = a[u].x ^ a[u].y ^ b[u].x ^ b[u].y;
            const uint32_t hi = a[u].z ^ a[u].w ^ b[u].z ^ b[u].w;
            __builtin_nontemporal_store(u32x2v{lo, hi}, codes + n);
            __builtin_nontemporal_store((uint8_t)(lo ^ hi ^ (lo >> 8) ^ (hi >> 16)), scales + n);
        }
    }
}

}  // namespace

// x: nblocks * 32 bytes (16-byte aligned); codes: nblocks * 8 bytes (8-byte aligned); scales: nblocks bytes.
// Returns 0, or the HIP error code of the launch (nothing is launched for nblocks == 0).
extern "C" int nvfp4_bench_stream(const void* x, int64_t nblocks, void* codes, void* scales, void* stream) {
    if (nblocks <= 0) return 0;
    const uint64_t per_wg = (uint64_t)kThreads * kUnroll;
    const uint64_t grid = ((uint64_t)nblocks + per_wg - 1) / per_wg;
    if (grid > 0x7FFFFFFFull) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(k_stream_blocks, dim3((uint32_t)grid), dim3(kThreads), 0, (hipStream_t)stream,
                       (const uint4*)x, (uint64_t)nblocks, (u32x2v*)codes, (uint8_t*)scales);
    return (int)hipGetLastError();
}

namespace {

// One wave that returns once `ticks` of the constant 100 MHz wall clock have passed: it holds the stream while
// the host queues the launches that are timed one by one, so that they run back to back.
__global__ void k_hold(uint64_t ticks) {
    const uint64_t t0 = wall_clock64();
    while (wall_clock64() - t0 < ticks) __builtin_amdgcn_s_sleep(8);
}

}  // namespace

// Holds `stream` for `microseconds` (at most one second).  Returns 0 or the HIP error code of the launch.
extern "C" int nvfp4_bench_hold(int64_t microseconds, void* stream) {
    if (microseconds < 0 || microseconds > 1000000) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(k_hold, dim3(1), dim3(64), 0, (hipStream_t)stream, (uint64_t)microseconds * 100u);
    return (int)hipGetLastError();
}
