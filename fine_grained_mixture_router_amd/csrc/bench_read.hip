// Benchmark instrumentation: one pass of 16-byte loads over a device buffer,
// the practical HBM read rate that the HBM-bound kernels are compared with
// (beside the nominal 8 TB/s).  Not part of the layer's computation.
//
// Each workgroup reads blocks of 1024 consecutive 16-byte vectors (four
// loads per thread, 4 KB apart), grid-strided over the buffer.  The loads
// feed an XOR that an empty asm statement consumes, so the compiler keeps
// every load and nothing is written.
#include "common.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p,
                                                          size_t nblocks) {
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (size_t b = blockIdx.x; b < nblocks; b += gridDim.x) {
        const u32x4* q = p + b * 1024 + threadIdx.x;
        const u32x4 v0 = q[0], v1 = q[256], v2 = q[512], v3 = q[768];
        acc ^= v0 ^ v1 ^ v2 ^ v3;
    }
    asm volatile("" :: "v"(acc.x ^ acc.y ^ acc.z ^ acc.w));
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, hipStream_t st) {
    const size_t nblocks = bytes / 16384;
    const unsigned grid = nblocks < 2048 ? (unsigned)nblocks : 2048u;
    stream_read_kernel<<<grid, 256, 0, st>>>(reinterpret_cast<const u32x4*>(buf), nblocks);
    return hipGetLastError();
}

}  // namespace moe
