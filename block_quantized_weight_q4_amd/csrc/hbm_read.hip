// hbm_read.hip -- a plain streaming read of a device buffer, the measured
// ceiling that the weight-streaming kernels are compared with.  Built as its
// own library (libkq_hbmread.so): it is a measuring stick, not part of the
// product interface in kq.h.
//
// Every lane reads 16-byte pieces, U of them in flight, in a grid-stride
// loop over the buffer, and folds them with XOR.  The result is stored only
// if it equals a value the caller passes and never expects, so the loads
// cannot be dropped while the kernel writes nothing in practice.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(256) void hbm_read_kernel(const u32x4* __restrict__ p, int64_t n16,
                                                       uint32_t never, uint32_t* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = p[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const u32x4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == never) sink[0] = acc;
}

}  // namespace

// Reads bytes (a multiple of 16, p 16-byte aligned) with `grid` workgroups
// of 256 threads and `unroll` (1, 2, 4 or 8) loads in flight per lane, on the
// given stream.  Returns 0, or -1 for invalid arguments, or the HIP error.
extern "C" int kq_hbm_read(const void* p, size_t bytes, int grid, int unroll, uint32_t never,
                           uint32_t* sink, void* stream) {
    if (!p || !sink || bytes == 0 || bytes % 16 || ((uintptr_t)p & 15) || grid <= 0) return -1;
    const int64_t n16 = (int64_t)(bytes / 16);
    hipStream_t s = (hipStream_t)stream;
    const u32x4* q = (const u32x4*)p;
    switch (unroll) {
    case 1: hipLaunchKernelGGL(hbm_read_kernel<1>, dim3(grid), dim3(256), 0, s, q, n16, never, sink); break;
    case 2: hipLaunchKernelGGL(hbm_read_kernel<2>, dim3(grid), dim3(256), 0, s, q, n16, never, sink); break;
    case 4: hipLaunchKernelGGL(hbm_read_kernel<4>, dim3(grid), dim3(256), 0, s, q, n16, never, sink); break;
    case 8: hipLaunchKernelGGL(hbm_read_kernel<8>, dim3(grid), dim3(256), 0, s, q, n16, never, sink); break;
    default: return -1;
    }
    return (int)hipGetLastError();
}
