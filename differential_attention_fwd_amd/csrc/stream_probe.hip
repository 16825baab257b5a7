// Streaming-read probe for gfx950: the rate at which this GPU reads a large buffer once, with the access pattern the
// decode kernels use (16-byte nontemporal loads, each wave instruction covering 1 KiB of contiguous memory).  It is
// measurement context for bench.py, next to the 8 TB/s nominal HBM peak; it computes nothing of the method and is not
// part of the library's ABI (built as its own libstreamprobe.so).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Grid-stride read of n16 16-byte chunks, UNROLL independent loads in flight per thread; the XOR of everything read
// goes to out[thread] so that no load is dead.
template <int UNROLL>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ buf, uint64_t n16,
                                                          unsigned* __restrict__ out) {
    const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    unsigned acc = 0;
    uint64_t i = tid;
    for (; i + (UNROLL - 1) * stride < n16; i += UNROLL * stride) {
        u32x4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(buf + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    out[tid] = acc;
}

}  // namespace

// Launches one read of `bytes` bytes (a multiple of 16, 16-byte aligned) with `blocks` workgroups of 256 threads and
// `unroll` in {1, 2, 4, 8} loads in flight per thread; `out` holds blocks * 256 unsigned.  Returns a hipError_t.
extern "C" int stream_read_probe(const void* buf, uint64_t bytes, unsigned* out, int blocks, int unroll,
                                 void* stream) {
    if (!buf || !out || blocks < 1 || (bytes & 15) || ((uintptr_t)buf & 15)) return (int)hipErrorInvalidValue;
    const uint64_t n16 = bytes / 16;
    const hipStream_t s = (hipStream_t)stream;
    const u32x4* b = (const u32x4*)buf;
    switch (unroll) {
        case 1: hipLaunchKernelGGL(stream_read_kernel<1>, dim3(blocks), dim3(256), 0, s, b, n16, out); break;
        case 2: hipLaunchKernelGGL(stream_read_kernel<2>, dim3(blocks), dim3(256), 0, s, b, n16, out); break;
        case 4: hipLaunchKernelGGL(stream_read_kernel<4>, dim3(blocks), dim3(256), 0, s, b, n16, out); break;
        case 8: hipLaunchKernelGGL(stream_read_kernel<8>, dim3(blocks), dim3(256), 0, s, b, n16, out); break;
        default: return (int)hipErrorInvalidValue;
    }
    return (int)hipGetLastError();
}
