// probe_kernels.hip -- plain streaming copy and read of a byte range, used to
// measure the HBM ceiling of the device and to calibrate the memory counters
// (FETCH_SIZE / WRITE_SIZE per byte moved).  Not part of the method.
#include "rssm_device.h"
#include "rssm_launch.h"

namespace rssm {

__global__ __launch_bounds__(256) void probe_copy_kernel(u32x4* __restrict__ dst,
                                                         const u32x4* __restrict__ src, long n16) {
    const long stride = (long)gridDim.x * blockDim.x;
    long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        const u32x4 b = __builtin_nontemporal_load(src + i + stride);
        const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
        __builtin_nontemporal_store(a, dst + i);
        __builtin_nontemporal_store(b, dst + i + stride);
        __builtin_nontemporal_store(c, dst + i + 2 * stride);
        __builtin_nontemporal_store(d, dst + i + 3 * stride);
    }
    for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* __restrict__ src, long n16,
                                                         float* sink) {
    const long stride = (long)gridDim.x * blockDim.x;
    long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        const u32x4 b = __builtin_nontemporal_load(src + i + stride);
        const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
        const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n16; i += stride) {
        const u32x4 a = __builtin_nontemporal_load(src + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    // keeps the loads alive; practically never taken
    if (acc == 0x7fc00001u) sink[0] = __uint_as_float(acc);
}

// One 32 KiB chunk per workgroup (8 non-temporal 16-byte loads per thread),
// then w16 16-byte plain stores: the read/write mix of a decode step.
__global__ __launch_bounds__(256) void probe_read_chunked_kernel(const u32x4* __restrict__ src,
                                                                 u32x4* __restrict__ dst, int w16, float* sink) {
    const long base = (long)blockIdx.x * 2048 + threadIdx.x;
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + base + u * 256);
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    if ((int)threadIdx.x < w16) dst[(long)blockIdx.x * w16 + threadIdx.x] = u32x4{acc, acc, acc, acc};
    if (acc == 0x7fc00001u) sink[0] = __uint_as_float(acc);
}

static int probe_grid(long n16) {
    long g = (n16 + 255) / 256;
    return (int)(g < 4096 ? (g > 0 ? g : 1) : 4096);
}

hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
    const long n16 = (long)(bytes / 16);
    hipLaunchKernelGGL(probe_copy_kernel, dim3(probe_grid(n16)), dim3(256), 0, s,
                       reinterpret_cast<u32x4*>(dst), reinterpret_cast<const u32x4*>(src), n16);
    return hipGetLastError();
}

hipError_t launch_probe_read(const void* src, size_t bytes, float* sink, hipStream_t s) {
    const long n16 = (long)(bytes / 16);
    hipLaunchKernelGGL(probe_read_kernel, dim3(probe_grid(n16)), dim3(256), 0, s,
                       reinterpret_cast<const u32x4*>(src), n16, sink);
    return hipGetLastError();
}

hipError_t launch_probe_read_chunked(const void* src, size_t bytes, void* dst, size_t write_bytes, float* sink,
                                     hipStream_t s) {
    const long chunks = (long)(bytes / 32768);
    hipLaunchKernelGGL(probe_read_chunked_kernel, dim3((unsigned)chunks), dim3(256), 0, s,
                       reinterpret_cast<const u32x4*>(src), reinterpret_cast<u32x4*>(dst),
                       (int)(write_bytes / 16), sink);
    return hipGetLastError();
}

}  // namespace rssm
