// probe.hip - a streaming read of device memory, as the bandwidth reference
// the decode kernels are measured against (not a step of the method).
//
// Every 16 bytes of the buffer are read once with non-temporal loads (as the
// split pass reads the cache), one load in flight per thread, over a grid
// that the dispatcher hands to whichever compute unit frees first; each
// block folds what it read into one word so the loads are not removed.
// One load per thread over 2048 blocks (8 MB in flight) read 160 MiB at 6.8
// TB/s on MI355X, against 6.5-6.6 TB/s for four loads per thread at its best
// block count (512); more bytes in flight than that lower the rate, so the
// caller sweeps the block count.
#include "common.hpp"
#include "kernels.hpp"

namespace otq {

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 1;

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4_t* __restrict__ buf, size_t n16,
                                                                    uint32_t* __restrict__ sink)
{
    const size_t stride = (size_t)gridDim.x * kProbeThreads;
    size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
        u32x4_t v[kProbeUnroll];
#pragma unroll
        for (int k = 0; k < kProbeUnroll; ++k) v[k] = __builtin_nontemporal_load(buf + i + k * stride);
#pragma unroll
        for (int k = 0; k < kProbeUnroll; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
    for (; i < n16; i += stride) {
        const u32x4_t v = __builtin_nontemporal_load(buf + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    // one word per block: the fold of its threads
    acc ^= __shfl_xor(acc, 1, 64) ^ __shfl_xor(acc, 2, 64);
    if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, hipStream_t stream)
{
    stream_read_kernel<<<blocks, kProbeThreads, 0, stream>>>(static_cast<const u32x4_t*>(buf), bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace otq
