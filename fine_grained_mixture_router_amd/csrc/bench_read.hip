// Benchmark instrumentation: one pass of 16-byte loads over a device buffer,
// the practical HBM read rate that the HBM-bound kernels are compared with
// (beside the nominal 8 TB/s).  Not part of the layer's computation.
//
// Each workgroup reads blocks of 2048 consecutive 16-byte vectors (eight
// loads per thread, 4 KB apart, nontemporal: the streaming policy that reads
// HBM fastest), grid-strided over the buffer.  The loads feed an XOR that an
// empty asm statement consumes, so the compiler keeps every load and nothing
// is written.
#include "common.h"

namespace moe {
namespace {

constexpr int kLoads = 8;
constexpr size_t kBlockBytes = (size_t)kLoads * 256 * 16;

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p,
                                                          size_t nblocks) {
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (size_t b = blockIdx.x; b < nblocks; b += gridDim.x) {
        const u32x4* q = p + b * (256 * kLoads) + threadIdx.x;
        u32x4 v[kLoads];
#pragma unroll
        for (int i = 0; i < kLoads; ++i) v[i] = __builtin_nontemporal_load(q + 256 * i);
#pragma unroll
        for (int i = 0; i < kLoads; ++i) acc ^= v[i];
    }
    asm volatile("" :: "v"(acc.x ^ acc.y ^ acc.z ^ acc.w));
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, hipStream_t st) {
    const size_t nblocks = bytes / kBlockBytes;
    const unsigned grid = nblocks < 4096 ? (unsigned)nblocks : 4096u;
    if (grid == 0) return hipSuccess;
    stream_read_kernel<<<grid, 256, 0, st>>>(reinterpret_cast<const u32x4*>(buf), nblocks);
    return hipGetLastError();
}

}  // namespace moe
