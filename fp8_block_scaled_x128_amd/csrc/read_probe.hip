// read_probe.hip -- a plain streaming read of a device buffer, for the benchmark's read floor: the
// time a launch needs just to read a given number of bytes from HBM on this part (launch,
// ramp-up and drain included), against which the decode-sized GEMMs, whose time is their operand
// stream, are compared.  Built into its own library (libreadprobe.so); the GEMM library does not
// contain it.
//
// Each workgroup of 256 threads reads one contiguous span of the buffer with 16-byte loads, DEPTH
// loads in flight per thread, folds the words together and writes one word per workgroup to
// `sink`, so the loads cannot be removed.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

template <int DEPTH>
__global__ __launch_bounds__(256) void read_probe_kernel(const v4u* __restrict__ buf, uint64_t n16,
                                                         uint64_t span16, uint32_t* __restrict__ sink) {
    const uint64_t begin = (uint64_t)blockIdx.x * span16;
    uint64_t end = begin + span16;
    if (end > n16) end = n16;
    v4u acc = {0u, 0u, 0u, 0u};
    uint64_t i = begin + threadIdx.x;
    for (; i + (DEPTH - 1) * 256 < end; i += DEPTH * 256) {
        v4u x[DEPTH];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) x[d] = buf[i + d * 256];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) acc ^= x[d];
    }
    for (; i < end; i += 256) acc ^= buf[i];
    const uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (v == 0x9E3779B9u) sink[blockIdx.x] = v;     // practically never taken; keeps the loads
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16) from `buf` (16-byte aligned, device) with `wgs` workgroups
// (each a contiguous span) and DEPTH = depth (4, 8 or 16) loads in flight per thread, on
// `stream`.  `sink` (device) holds at least `wgs` uint32.  Returns 0, or -1 on a bad argument or
// a failed launch.
int read_probe(const void* buf, uint64_t bytes, int wgs, int depth, void* sink, void* stream) {
    if (!buf || !sink || wgs <= 0 || (bytes & 15) != 0 || ((uintptr_t)buf & 15) != 0) return -1;
    const uint64_t n16 = bytes / 16;
    const uint64_t span16 = ((n16 + wgs - 1) / wgs + 255) / 256 * 256;
    const dim3 grid((unsigned)wgs), block(256);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const v4u* b = static_cast<const v4u*>(buf);
    uint32_t* k = static_cast<uint32_t*>(sink);
    switch (depth) {
        case 4: hipLaunchKernelGGL(read_probe_kernel<4>, grid, block, 0, s, b, n16, span16, k); break;
        case 8: hipLaunchKernelGGL(read_probe_kernel<8>, grid, block, 0, s, b, n16, span16, k); break;
        case 16: hipLaunchKernelGGL(read_probe_kernel<16>, grid, block, 0, s, b, n16, span16, k); break;
        default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
