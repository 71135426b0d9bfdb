// Streaming 16-byte copy: the attainable-bandwidth reference the benchmark
// sets beside the HBM-bound convolution kernels.  A grid of a few
// workgroups per compute unit strides over the buffer; per step a thread
// requests U 16-byte loads (consecutive threads on consecutive pieces, so a
// wave moves 1 KB per load instruction) before it stores any of them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/conv2d_probe.h"

namespace {

constexpr int kT = 256;
constexpr int U = 4;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kT) void probe_copy_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src,
                                                        int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kT * U;
    for (int64_t base = (int64_t)blockIdx.x * kT * U + threadIdx.x; base < n; base += stride) {
        u32x4 v[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int64_t j = base + (int64_t)i * kT;
            v[i] = j < n ? __builtin_nontemporal_load(src + j) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int64_t j = base + (int64_t)i * kT;
            if (j < n) __builtin_nontemporal_store(v[i], dst + j);
        }
    }
}

}  // namespace

extern "C" conv_status_t conv2d_probe_copy(void* dst, const void* src, int64_t bytes, void* stream) {
    if (!dst || !src || bytes < 0 || bytes % 16 || (uintptr_t)dst % 16 || (uintptr_t)src % 16)
        return CONV_ERR_INVALID_ARG;
    const uintptr_t d = (uintptr_t)dst, s = (uintptr_t)src;
    if (d < s + (uintptr_t)bytes && s < d + (uintptr_t)bytes && bytes > 0) return CONV_ERR_ALIAS;
    const int64_t n = bytes / 16;
    if (n == 0) return CONV_OK;
    int cus = 256, dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
        cus = v;
    const int64_t need = (n + kT * U - 1) / (kT * U);
    const int64_t cap = (int64_t)cus * 8;
    const uint32_t grid = (uint32_t)(need < cap ? need : cap);
    u32x4* dp = (u32x4*)dst;
    const u32x4* sp = (const u32x4*)src;
    int64_t nn = n;
    void* args[] = {&dp, (void*)&sp, &nn};
    return hipLaunchKernel((const void*)probe_copy_kernel, dim3(grid), dim3(kT), args, 0, (hipStream_t)stream) ==
                   hipSuccess
               ? CONV_OK
               : CONV_ERR_HIP;
}
