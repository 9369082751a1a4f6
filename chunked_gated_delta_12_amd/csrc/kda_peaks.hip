// kda_peaks.hip -- on-device reference measurements (declared in
// include/kda_peaks.h): a streaming copy, a dense bf16 matrix-core loop and the
// device's description.  Built into libkda_peaks.so, separate from libkda.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "kda_peaks.h"

namespace {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

constexpr int kCopyThreads = 256;
constexpr int kCopyPerThread = 4;

// Each thread moves kCopyPerThread 16-byte units spaced a workgroup apart, all
// loads issued before the stores.  n counts 16-byte units.
__global__ __launch_bounds__(kCopyThreads) void copy_kernel(const uint4* __restrict__ src,
                                                             uint4* __restrict__ dst, size_t n) {
    const size_t base = (size_t)blockIdx.x * (kCopyThreads * kCopyPerThread) + threadIdx.x;
    uint4 r[kCopyPerThread];
#pragma unroll
    for (int j = 0; j < kCopyPerThread; ++j) {
        const size_t i = base + (size_t)j * kCopyThreads;
        if (i < n) r[j] = src[i];
    }
#pragma unroll
    for (int j = 0; j < kCopyPerThread; ++j) {
        const size_t i = base + (size_t)j * kCopyThreads;
        if (i < n) dst[i] = r[j];
    }
}

// 8 independent accumulation chains per wavefront keep the matrix core busy
// while each instruction's result is pending.
__global__ __launch_bounds__(256) void mfma_kernel(float* __restrict__ sink, int iters) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(0.001f * (float)(lane + i));
        b[i] = (__bf16)(0.002f * (float)(63 - lane + i));
    }
    f32x4 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {   // distinct start values: eight distinct chains
        const float x = 0.01f * (float)(c * 64 + lane);
        acc[c] = f32x4{x, -x, 0.5f * x, 2.f * x};
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    sink[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" {

int kda_peaks_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (!src || !dst || bytes == 0 || (bytes & 15u)) return 1;
    if (((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u)) return 1;
    const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
    if (s0 < d0 + bytes && d0 < s0 + bytes) return 1;
    const size_t n = bytes / 16;
    const size_t per_block = (size_t)kCopyThreads * kCopyPerThread;
    const size_t blocks = (n + per_block - 1) / per_block;
    if (blocks > 0x7fffffffULL) return 1;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), (const uint4*)src, (uint4*)dst, n);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int kda_peaks_mfma_bf16(float* sink, int workgroups, int iters, void* stream) {
    if (!sink || workgroups < 1 || iters < 1 || ((uintptr_t)sink & 3u)) return 1;
    hipLaunchKernelGGL(mfma_kernel, dim3((unsigned)workgroups), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), sink, iters);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

int kda_peaks_device(int device, kda_device_info* info) {
    if (!info || device < 0) return 1;
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, device) != hipSuccess) return 2;
    memset(info, 0, sizeof(*info));
    strncpy(info->name, p.name, sizeof(info->name) - 1);
    strncpy(info->arch, p.gcnArchName, sizeof(info->arch) - 1);
    info->compute_units = p.multiProcessorCount;
    info->clock_khz = p.clockRate;
    info->memory_clock_khz = p.memoryClockRate;
    info->memory_bus_bits = p.memoryBusWidth;
    info->l2_bytes = p.l2CacheSize;
    info->total_bytes = (long long)p.totalGlobalMem;
    info->lds_bytes_per_cu = (int)p.maxSharedMemoryPerMultiProcessor;
    info->warp_size = p.warpSize;
    return 0;
}

}  // extern "C"
