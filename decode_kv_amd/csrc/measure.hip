// csa2_stream_read: a plain read of a buffer with the launch shape of the Full
// scan's scoring kernel (one 512-thread workgroup per 64 KiB, every thread
// issuing its eight 16-byte loads before using any), so that the scan's
// bandwidth can be set against what a kernel that only reads the same bytes
// reaches on the same part.  Not a step of the method: it computes nothing
// but an XOR of what it read, one word per workgroup.
#include "abi_common.h"
#include "common.h"

namespace csa2 {

constexpr int kReadThreads = 512;
constexpr int kReadLoads = 8;
constexpr size_t kReadChunk = (size_t)kReadThreads * kReadLoads * 16;   // 64 KiB per workgroup

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4* __restrict__ src,
                                                                   size_t n16,
                                                                   uint32_t* __restrict__ sink) {
    // wave w reads 8 KiB: lane l takes 16-byte pieces l, l + 64, ... of it
    const int wave = threadIdx.x / kWave, l = lane_id();
    const size_t first = (size_t)blockIdx.x * (kReadChunk / 16) + (size_t)wave * kWave * kReadLoads;
    u32x4 v[kReadLoads];
#pragma unroll
    for (int u = 0; u < kReadLoads; ++u) {
        const size_t i = first + (size_t)u * kWave + l;
        v[u] = i < n16 ? src[i] : u32x4{0u, 0u, 0u, 0u};
    }
    uint32_t x = 0;
#pragma unroll
    for (int u = 0; u < kReadLoads; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    x = (uint32_t)wave_sum((float)(x & 0xFFFF));             // keeps every load live
    __shared__ uint32_t s_x[kReadThreads / kWave];
    if (l == 0) s_x[wave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t y = 0;
#pragma unroll
        for (int i = 0; i < kReadThreads / kWave; ++i) y ^= s_x[i];
        sink[blockIdx.x] = y;
    }
}

}  // namespace csa2

using namespace csa2;

extern "C" size_t csa2_stream_read_sink_words(size_t bytes) {
    return (bytes + kReadChunk - 1) / kReadChunk;
}

extern "C" int csa2_stream_read(const void* src, size_t bytes, unsigned int* sink,
                                size_t sink_words, void* stream) {
    if (bytes == 0) return CSA2_OK;
    if (!src || !sink) return fail(CSA2_ERR_INVALID, "csa2_stream_read: null pointer");
    if (!aligned(src, 16) || bytes % 16 != 0 || !aligned(sink, 4))
        return fail(CSA2_ERR_INVALID, "csa2_stream_read: misaligned pointer or size");
    const size_t grid = csa2_stream_read_sink_words(bytes);
    if (sink_words < grid)
        return fail(CSA2_ERR_WORKSPACE, "csa2_stream_read: sink needs %zu words", grid);
    if (grid > 0x7FFFFFFFu) return fail(CSA2_ERR_UNSUPPORTED, "csa2_stream_read: too large");
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kReadThreads), 0,
                       reinterpret_cast<hipStream_t>(stream),
                       reinterpret_cast<const u32x4*>(src), bytes / 16, sink);
    return launch_status("csa2_stream_read launch");
}
