// Measurement helpers, not steps of the method.
//
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

// ---- the cost of a kernel boundary and of handing partial results over ---------
// csa2_empty_kernel: a kernel that does nothing, to time a graph node.
// csa2_handoff: groups x splits workgroups each write a partial of kHoPer
// floats; each group's kHoPer outputs are the sums over its splits.  Mode 0
// merges in a second kernel; modes 1 and 2 merge in the same kernel after a
// per-group arrival counter (1: partials stored through to memory with
// device-scope relaxed atomic stores and read back the same way; 2: plain
// stores and loads between device-scope release and acquire fences).  In
// modes 1 and 2 every workgroup of a group waits for the others, so the
// launch keeps at most 256 workgroups (all resident at once), and the wait is
// bounded: a workgroup that gives up writes NaN.
constexpr int kHoThreads = 256;
constexpr int kHoPer = 8192;
constexpr int kHoMaxWgs = 256;
constexpr long long kHoSpin = 1ll << 16;

__global__ void empty_kernel() {}

__device__ __forceinline__ bool ho_place(int groups, int splits, int& g, int& s) {
    const int xid = blockIdx.x & 7, xslot = blockIdx.x >> 3;   // workgroup i on XCD i mod 8
    const int lp = xslot / splits;
    s = xslot - lp * splits;
    g = lp * 8 + xid;
    return g < groups;
}

__device__ __forceinline__ float ho_value(float v, int s, int i) { return v + s + i * 1e-6f; }

__global__ __launch_bounds__(kHoThreads) void ho_write_kernel(float* part, int groups, int splits,
                                                              float v) {
    int g, s;
    if (!ho_place(groups, splits, g, s)) return;
    float* p = part + ((size_t)g * splits + s) * kHoPer;
    for (int i = threadIdx.x; i < kHoPer; i += kHoThreads) p[i] = ho_value(v, s, i);
}

__global__ __launch_bounds__(128) void ho_merge_kernel(const float* part, float* out, int groups,
                                                       int splits) {
    const int xid = blockIdx.x & 7, xslot = blockIdx.x >> 3;   // 16 workgroups per group
    const int lp = xslot / 16, sl = xslot - lp * 16;
    const int g = lp * 8 + xid;
    if (g >= groups) return;
    const int c0 = sl * (kHoPer / 16);
    for (int c = c0 + threadIdx.x; c < c0 + kHoPer / 16; c += 128) {
        float acc = 0.f;
        for (int s = 0; s < splits; ++s) acc += part[((size_t)g * splits + s) * kHoPer + c];
        out[(size_t)g * kHoPer + c] = acc;
    }
}

template <int MODE>
__global__ __launch_bounds__(kHoThreads) void ho_fused_kernel(float* part, unsigned* cnt,
                                                              float* out, int groups, int splits,
                                                              float v) {
    int g, s;
    if (!ho_place(groups, splits, g, s)) return;
    float* p = part + ((size_t)g * splits + s) * kHoPer;
    for (int i = threadIdx.x; i < kHoPer; i += kHoThreads) {
        if (MODE == 1)
            __hip_atomic_store(p + i, ho_value(v, s, i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
            p[i] = ho_value(v, s, i);
    }
    if (MODE == 1) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    else __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    __shared__ int s_ok;
    if (threadIdx.x == 0) {
        __hip_atomic_fetch_add(cnt + 2 * g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        long long it = 0;
        while (__hip_atomic_load(cnt + 2 * g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                   (unsigned)splits &&
               it < kHoSpin)
            ++it;
        s_ok = it < kHoSpin;
    }
    __syncthreads();
    if (MODE == 1) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    else __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    const int w = (kHoPer + splits - 1) / splits;              // this workgroup's slice
    const int c1 = min(kHoPer, (s + 1) * w);
    for (int c = s * w + threadIdx.x; c < c1; c += kHoThreads) {
        float acc = 0.f;
        for (int t = 0; t < splits; ++t) {
            const float* q = part + ((size_t)g * splits + t) * kHoPer + c;
            acc += MODE == 1 ? __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : *q;
        }
        out[(size_t)g * kHoPer + c] = s_ok ? acc : __builtin_nanf("");
    }
    __syncthreads();
    if (threadIdx.x == 0) {                                    // the last to leave resets
        const unsigned d =
            __hip_atomic_fetch_add(cnt + 2 * g + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (d == (unsigned)splits - 1) {
            __hip_atomic_store(cnt + 2 * g, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(cnt + 2 * g + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

static size_t ho_part_bytes(int groups, int splits) {
    return round_up((size_t)groups * splits * kHoPer * 4, 256);
}

}  // namespace csa2

using namespace csa2;

extern "C" int csa2_empty_kernel(void* stream) {
    hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, reinterpret_cast<hipStream_t>(stream));
    return launch_status("csa2_empty_kernel launch");
}

extern "C" size_t csa2_handoff_scratch_bytes(int groups, int splits) {
    if (groups < 1 || splits < 1) return 0;
    return ho_part_bytes(groups, splits) + 2 * 4 * (size_t)groups;
}

extern "C" int csa2_handoff(int mode, int groups, int splits, float value, void* scratch,
                            size_t scratch_bytes, float* out, void* stream) {
    const char* fn = "csa2_handoff";
    if (mode < 0 || mode > 2 || groups < 1 || splits < 1 || splits > kHoPer)
        return fail(CSA2_ERR_INVALID, "%s: mode, groups or splits out of range", fn);
    if (!scratch || !out || !aligned(scratch, 256) || !aligned(out, 4))
        return fail(CSA2_ERR_INVALID, "%s: null or misaligned pointer", fn);
    if (scratch_bytes < csa2_handoff_scratch_bytes(groups, splits))
        return fail(CSA2_ERR_WORKSPACE, "%s: scratch needs %zu bytes", fn,
                    csa2_handoff_scratch_bytes(groups, splits));
    const int lanes = (groups + 7) / 8;                         // group slots per XCD
    const long long wgs = 8ll * lanes * splits;
    if (mode > 0 && wgs > kHoMaxWgs)
        return fail(CSA2_ERR_UNSUPPORTED, "%s: modes 1 and 2 keep at most %d workgroups", fn,
                    kHoMaxWgs);
    if (wgs > 0x7FFFFFFFll) return fail(CSA2_ERR_UNSUPPORTED, "%s: too many workgroups", fn);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    float* part = reinterpret_cast<float*>(scratch);
    unsigned* cnt = reinterpret_cast<unsigned*>(reinterpret_cast<char*>(scratch) +
                                                ho_part_bytes(groups, splits));
    const dim3 grid((unsigned)wgs), blk(kHoThreads);
    if (mode == 0) {
        hipLaunchKernelGGL(ho_write_kernel, grid, blk, 0, s, part, groups, splits, value);
        if (int e = launch_status(fn)) return e;
        hipLaunchKernelGGL(ho_merge_kernel, dim3(8 * lanes * 16), dim3(128), 0, s, part, out,
                           groups, splits);
    } else if (mode == 1) {
        hipLaunchKernelGGL(ho_fused_kernel<1>, grid, blk, 0, s, part, cnt, out, groups, splits,
                           value);
    } else {
        hipLaunchKernelGGL(ho_fused_kernel<2>, grid, blk, 0, s, part, cnt, out, groups, splits,
                           value);
    }
    return launch_status(fn);
}

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
