// Test infrastructure: a kernel that holds CUs for a fixed time, standing in for a kernel on
// another stream (a collective, for instance) that occupies CUs while a single-pass quantization
// waits at its grid barrier. `grid` workgroups of 64 threads, each with `lds` bytes of dynamic
// LDS, spin on the 100 MHz real-time counter for `us` microseconds and then exit.
#include <hip/hip_runtime.h>
#include <stdint.h>

__global__ void holder_kernel(uint32_t ticks, uint32_t *sink) {
    extern __shared__ uint32_t buf[];
    buf[threadIdx.x] = threadIdx.x;                 // 64 words: the smallest lds accepted is 256 B
    const uint64_t start = __builtin_amdgcn_s_memrealtime();
    uint32_t acc = 0;
    while (__builtin_amdgcn_s_memrealtime() - start < ticks) {
        acc += buf[(threadIdx.x + acc) & 63u];
        __builtin_amdgcn_s_sleep(8);
    }
    if (acc == 0xFFFFFFFFu) sink[0] = acc;          // keeps the loop; practically never stores
}

// Returns 0, or 1 for arguments out of range, 2 for a launch error.
extern "C" int holder_launch(int grid, int lds, int us, uint32_t *sink, hipStream_t s) {
    if (grid < 1 || grid > 4096 || lds < 256 || lds > 64 * 1024 || us < 0 || us > 100000 || !sink) return 1;
    hipLaunchKernelGGL(holder_kernel, dim3(grid), dim3(64), (size_t)lds, s, (uint32_t)us * 100u, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
