// csa2_kv_append_fp4: quantise bf16 latent rows into the FP4 E2M1 cache with
// one E8M0 scale per 32 elements.  ("DeepSeek V4.1-Flash 552B runs like 16B
// (CED)", "Act 3": the main KV cache is kept in 4-bit floating point; the
// block rule is that of OCP MX v1.0.)
//
// One wavefront per row: lane l owns elements [8l, 8l+8) of a 512-wide chunk
// (one 16-byte load), four lanes own one 32-element block.  The block amax is
// reduced over those four lanes; rounding is done in exact integer arithmetic
// on the bf16 bits, so the output bytes do not depend on float modes.
#include "abi_common.h"
#include "common.h"

namespace csa2 {

constexpr int kAppendThreads = 256;  // 4 rows per workgroup

// E2M1 code (0..7) of |x| / 2^(b-127) for a bf16 magnitude `mag`, rounding to
// nearest with ties to the even code and saturating at 6.
__device__ __forceinline__ uint32_t e2m1_code(uint32_t mag, int b) {
    const int e = (int)(mag >> 7);
    const uint32_t sig = e ? (0x80u | (mag & 0x7Fu)) : (mag & 0x7Fu);
    if (sig == 0) return 0;
    // 4*y = sig * 2^t with t = max(e,1) - b - 5
    const int t = (e ? e : 1) - b - 5;
    uint32_t y4;
    bool sticky;
    if (t >= 5) {
        return 7;  // 4*y >= 32 > 20
    } else if (t >= 0) {
        y4 = sig << t;
        sticky = false;
    } else if (t > -9) {
        y4 = sig >> (-t);
        sticky = (sig & ((1u << (-t)) - 1u)) != 0;
    } else {
        y4 = 0;
        sticky = true;  // sig != 0
    }
    // midpoints in units of 1/4: 0.25 0.75 1.25 1.75 2.5 3.5 5
    const uint32_t s = sticky ? 1u : 0u;
    uint32_t c = 0;
    c += (y4 > 1u) | ((y4 == 1u) & s);
    c += (y4 > 3u) | ((y4 == 3u) & s);
    c += (y4 > 5u) | ((y4 == 5u) & s);
    c += (y4 > 7u) | ((y4 == 7u) & s);
    c += (y4 > 10u) | ((y4 == 10u) & s);
    c += (y4 > 14u) | ((y4 == 14u) & s);
    c += (y4 > 20u) | ((y4 == 20u) & s);
    const bool tie = !sticky && (y4 == 1u || y4 == 3u || y4 == 5u || y4 == 7u || y4 == 10u ||
                                 y4 == 14u || y4 == 20u);
    if (tie) c += (c & 1u);  // an exact midpoint goes to the even code
    return c;
}

// Lane l's 16-byte piece of the 512-wide chunk at `base` of a row of D bf16
// values (elements base + 8l .. + 7; zeros past D, D % 32 == 0).
__device__ __forceinline__ u32x4 load_chunk(const uint16_t* __restrict__ xr, int D, int base) {
    const int e0 = base + 8 * lane_id();
    return e0 < D ? *reinterpret_cast<const u32x4*>(xr + e0) : u32x4{0u, 0u, 0u, 0u};
}

// Quantise and store one 512-wide chunk of a row with one wavefront: lane l
// owns elements [8l, 8l+8) of the chunk (its piece v), four lanes one
// 32-element block.
__device__ __forceinline__ void quantise_chunk(u32x4 v, int D, int base,
                                               uint8_t* __restrict__ codes_row,
                                               uint8_t* __restrict__ scale_row) {
    const int l = lane_id();
    {
        const int e0 = base + 8 * l;
        const bool active = e0 < D;  // D % 32 == 0: whole 4-lane groups
        uint32_t h[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            h[2 * j] = v[j] & 0xFFFFu;
            h[2 * j + 1] = v[j] >> 16;
        }
        uint32_t amax = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = max(amax, h[j] & 0x7FFFu);
        amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
        amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
        // E8M0 byte: biased exponent of amax minus 2, clamped at 0 (zero and
        // subnormal blocks).  Finite bf16 keeps it <= 252.
        const int ef = (int)(amax >> 7);
        const int b = ef > 2 ? ef - 2 : 0;
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t c = e2m1_code(h[j] & 0x7FFFu, b) | ((h[j] >> 12) & 8u);
            word |= c << (4 * j);
        }
        if (active) {
            *reinterpret_cast<uint32_t*>(codes_row + e0 / 2) = word;
            if ((l & 3) == 0) scale_row[e0 / 32] = (uint8_t)b;
        }
    }
}

// Quantise one row of D bf16 values with one wavefront, chunk by chunk.
__device__ __forceinline__ void quantise_row_fp4(const uint16_t* __restrict__ xr, int D,
                                                 uint8_t* __restrict__ codes_row,
                                                 uint8_t* __restrict__ scale_row) {
    for (int base = 0; base < D; base += 512)
        quantise_chunk(load_chunk(xr, D, base), D, base, codes_row, scale_row);
}

__global__ __launch_bounds__(kAppendThreads) void kv_append_fp4_kernel(
    const uint16_t* __restrict__ x, const long long* __restrict__ dst_row, int n, int D,
    uint8_t* __restrict__ kv_fp4, uint8_t* __restrict__ kv_scale) {
    const int wave = threadIdx.x / kWave;
    const long long r = (long long)blockIdx.x * (kAppendThreads / kWave) + wave;
    if (r >= n) return;
    const long long dst = dst_row[r];
    quantise_row_fp4(x + r * (long long)D, D, kv_fp4 + dst * (long long)(D / 2),
                     kv_scale + dst * (long long)(D / 32));
}

// One workgroup of 16 waves per sequence b: the token's FP4 row of every
// layer (wave w takes layers w, w + 16, ...) and its index key go to row
// row_off[b] + len[b]; after a barrier, thread 0 advances len[b].  Only this
// workgroup reads or writes len[b], so the old length is read before the new
// one is stored.  A wave issues the loads of its first two rows before it
// quantises either, so the step pays one load round trip.
constexpr int kTokenThreads = 1024;

__global__ __launch_bounds__(kTokenThreads) void append_token_kernel(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ key_rows,
    const long long* __restrict__ row_off, int* __restrict__ len, int B, int n_layers,
    long long layer_rows, int D, uint8_t* __restrict__ kv_fp4, uint8_t* __restrict__ kv_scale,
    int8_t* __restrict__ keys) {
    const int b = blockIdx.x;
    const int wave = threadIdx.x / kWave;
    const int L = len[b];
    const long long row = row_off[b] + L;
    if (threadIdx.x < kDk / 16)                       // the 64-byte index key, 16 bytes a thread
        *reinterpret_cast<u32x4*>(keys + row * kDk + 16 * threadIdx.x) =
            *reinterpret_cast<const u32x4*>(key_rows + (size_t)b * kDk + 16 * threadIdx.x);
    constexpr int NW = kTokenThreads / kWave;
    const int l0 = wave, l1 = wave + NW;
    const uint16_t* x0 = x + ((size_t)l0 * B + b) * D;
    const uint16_t* x1 = x + ((size_t)l1 * B + b) * D;
    const u32x4 v0 = l0 < n_layers ? load_chunk(x0, D, 0) : u32x4{0u, 0u, 0u, 0u};
    const u32x4 v1 = l1 < n_layers ? load_chunk(x1, D, 0) : u32x4{0u, 0u, 0u, 0u};
    auto finish = [&](int layer, const uint16_t* xr, u32x4 v) {
        const long long dst = layer * layer_rows + row;
        uint8_t* cr = kv_fp4 + dst * (long long)(D / 2);
        uint8_t* sr = kv_scale + dst * (long long)(D / 32);
        quantise_chunk(v, D, 0, cr, sr);
        for (int base = 512; base < D; base += 512)
            quantise_chunk(load_chunk(xr, D, base), D, base, cr, sr);
    };
    if (l0 < n_layers) finish(l0, x0, v0);
    if (l1 < n_layers) finish(l1, x1, v1);
    for (int layer = wave + 2 * NW; layer < n_layers; layer += NW)
        quantise_row_fp4(x + ((size_t)layer * B + b) * D, D, kv_fp4 + (layer * layer_rows + row) * (long long)(D / 2),
                         kv_scale + (layer * layer_rows + row) * (long long)(D / 32));
    __syncthreads();                                  // every thread has read len[b]
    if (threadIdx.x == 0) len[b] = L + 1;
}

}  // namespace csa2

using namespace csa2;

extern "C" int csa2_kv_append_fp4(const void* x_bf16, const long long* dst_row, int n, int D,
                                  unsigned char* kv_fp4, unsigned char* kv_scale, void* stream) {
    if (n < 0) return fail(CSA2_ERR_INVALID, "csa2_kv_append_fp4: n < 0");
    if (n == 0) return CSA2_OK;
    if (!x_bf16 || !dst_row || !kv_fp4 || !kv_scale)
        return fail(CSA2_ERR_INVALID, "csa2_kv_append_fp4: null pointer");
    if (D <= 0 || D % 32 != 0) return fail(CSA2_ERR_INVALID, "csa2_kv_append_fp4: D %% 32 != 0");
    if (!aligned(x_bf16, 16) || !aligned(kv_fp4, 4) || !aligned(dst_row, 8))
        return fail(CSA2_ERR_INVALID, "csa2_kv_append_fp4: misaligned pointer");
    const int rows_per_block = kAppendThreads / kWave;
    const unsigned grid = (unsigned)((n + rows_per_block - 1) / rows_per_block);
    hipLaunchKernelGGL(kv_append_fp4_kernel, dim3(grid), dim3(kAppendThreads), 0,
                       reinterpret_cast<hipStream_t>(stream),
                       reinterpret_cast<const uint16_t*>(x_bf16), dst_row, n, D, kv_fp4,
                       kv_scale);
    return launch_status("csa2_kv_append_fp4 launch");
}

extern "C" int csa2_append_token(const void* x_bf16, const signed char* key_rows,
                                 const long long* row_off, int* len, int B, int n_layers,
                                 long long layer_rows, int D, int Dk, unsigned char* kv_fp4,
                                 unsigned char* kv_scale, signed char* keys, void* stream) {
    if (B < 0 || n_layers < 0 || layer_rows < 0)
        return fail(CSA2_ERR_INVALID, "csa2_append_token: negative size");
    if (B == 0) return CSA2_OK;
    if (!key_rows || !row_off || !len || !keys || (n_layers > 0 && (!x_bf16 || !kv_fp4 || !kv_scale)))
        return fail(CSA2_ERR_INVALID, "csa2_append_token: null pointer");
    if (Dk != kDk) return fail(CSA2_ERR_UNSUPPORTED, "csa2_append_token: Dk must be 64");
    if (D <= 0 || D % 32 != 0) return fail(CSA2_ERR_INVALID, "csa2_append_token: D %% 32 != 0");
    if (B > 65535) return fail(CSA2_ERR_UNSUPPORTED, "csa2_append_token: B > 65535");
    if (!aligned(x_bf16, 16) || !aligned(key_rows, 16) || !aligned(keys, 16) ||
        !aligned(kv_fp4, 4) || !aligned(row_off, 8) || !aligned(len, 4))
        return fail(CSA2_ERR_INVALID, "csa2_append_token: misaligned pointer");
    hipLaunchKernelGGL(append_token_kernel, dim3(B), dim3(kTokenThreads), 0,
                       reinterpret_cast<hipStream_t>(stream),
                       reinterpret_cast<const uint16_t*>(x_bf16),
                       reinterpret_cast<const int8_t*>(key_rows), row_off, len, B, n_layers,
                       layer_rows, D, kv_fp4, kv_scale, reinterpret_cast<int8_t*>(keys));
    return launch_status("csa2_append_token launch");
}
