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

// One workgroup of 16 waves per sequence b appends its n tokens: token j's
// FP4 row of every layer (items (j, layer), wave w taking items w, w + 16,
// ...) and its index key go to row row_off[b] + len[b] + j; after a barrier,
// thread 0 advances len[b] by n.  Only this workgroup reads or writes len[b],
// so the old length is read before the new one is stored.  A wave issues the
// loads of its first two rows before it reads the length and quantises
// either, so a one-token step pays one load round trip.
constexpr int kTokenThreads = 1024;

__global__ __launch_bounds__(kTokenThreads) void append_token_kernel(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ key_rows,
    const long long* __restrict__ row_off, int* __restrict__ len, int B, int n, int n_layers,
    long long layer_rows, int D, uint8_t* __restrict__ kv_fp4, uint8_t* __restrict__ kv_scale,
    int8_t* __restrict__ keys) {
    const int b = blockIdx.x;
    const int wave = threadIdx.x / kWave;
    constexpr int NW = kTokenThreads / kWave;
    const int items = n * n_layers;                   // (token, layer) rows of this sequence
    auto src = [&](int i) {                           // x is [n][n_layers][B][D]
        return x + ((size_t)i * B + b) * D;
    };
    // the wave's first two rows are loaded before the length arrives: their
    // round trip overlaps the length's
    u32x4 v0 = wave < items ? load_chunk(src(wave), D, 0) : u32x4{0u, 0u, 0u, 0u};
    u32x4 v1 = wave + NW < items ? load_chunk(src(wave + NW), D, 0) : u32x4{0u, 0u, 0u, 0u};
    const int L = len[b];
    const long long row0 = row_off[b] + L;
    for (int i = threadIdx.x; i < n * (kDk / 16); i += kTokenThreads) {   // 16 key bytes a thread
        const int j = i / (kDk / 16), c = i % (kDk / 16);
        *reinterpret_cast<u32x4*>(keys + (row0 + j) * kDk + 16 * c) =
            *reinterpret_cast<const u32x4*>(key_rows + ((size_t)j * B + b) * kDk + 16 * c);
    }
    auto finish = [&](int i, u32x4 v) {
        const int j = i / n_layers, layer = i - j * n_layers;
        const long long dst = layer * layer_rows + row0 + j;
        uint8_t* cr = kv_fp4 + dst * (long long)(D / 2);
        uint8_t* sr = kv_scale + dst * (long long)(D / 32);
        quantise_chunk(v, D, 0, cr, sr);
        for (int base = 512; base < D; base += 512)
            quantise_chunk(load_chunk(src(i), D, base), D, base, cr, sr);
    };
    for (int i0 = wave; i0 < items; i0 += 2 * NW) {  // two rows' loads in flight
        const int i1 = i0 + NW;
        if (i0 > wave) {
            v0 = load_chunk(src(i0), D, 0);
            v1 = i1 < items ? load_chunk(src(i1), D, 0) : u32x4{0u, 0u, 0u, 0u};
        }
        finish(i0, v0);
        if (i1 < items) finish(i1, v1);
    }
    __syncthreads();                                  // every thread has read len[b]
    if (threadIdx.x == 0) len[b] = L + n;
}

// Many rows per sequence (a replayed window: n tokens times every layer):
// the rows are spread over workgroups (x, b) of kWideItems (token, layer)
// items each, which all read len[b]; the index keys and the length advance
// follow in append_keys_len_kernel, launched after it on the same stream.
constexpr int kWideItems = 64;
constexpr int kWideThreads = 1024;    // 16 waves x 4 items, every load issued first

__global__ __launch_bounds__(kWideThreads) void append_rows_wide_kernel(
    const uint16_t* __restrict__ x, const long long* __restrict__ row_off,
    const int* __restrict__ len, int B, int n, int n_layers, long long layer_rows, int D,
    uint8_t* __restrict__ kv_fp4, uint8_t* __restrict__ kv_scale) {
    const int b = blockIdx.y;
    const int wave = threadIdx.x / kWave;
    constexpr int NW = kWideThreads / kWave;
    constexpr int PER = kWideItems / NW;
    const long long row0 = row_off[b] + len[b];
    const int items = n * n_layers;
    const int first = blockIdx.x * kWideItems + wave;
    u32x4 v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int i = first + u * NW;
        v[u] = i < items ? load_chunk(x + ((size_t)i * B + b) * D, D, 0) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int i = first + u * NW;
        if (i >= items) break;
        const int j = i / n_layers, layer = i - j * n_layers;
        const long long dst = layer * layer_rows + row0 + j;
        uint8_t* cr = kv_fp4 + dst * (long long)(D / 2);
        uint8_t* sr = kv_scale + dst * (long long)(D / 32);
        quantise_chunk(v[u], D, 0, cr, sr);
        for (int base = 512; base < D; base += 512)
            quantise_chunk(load_chunk(x + ((size_t)i * B + b) * D, D, base), D, base, cr, sr);
    }
}

__global__ __launch_bounds__(256) void append_keys_len_kernel(
    const int8_t* __restrict__ key_rows, const long long* __restrict__ row_off,
    int* __restrict__ len, int B, int n, int8_t* __restrict__ keys) {
    const int b = blockIdx.x;
    const int L = len[b];
    const long long row0 = row_off[b] + L;
    for (int i = threadIdx.x; i < n * (kDk / 16); i += 256) {
        const int j = i / (kDk / 16), c = i % (kDk / 16);
        *reinterpret_cast<u32x4*>(keys + (row0 + j) * kDk + 16 * c) =
            *reinterpret_cast<const u32x4*>(key_rows + ((size_t)j * B + b) * kDk + 16 * c);
    }
    __syncthreads();                                  // every thread has read len[b]
    if (threadIdx.x == 0) len[b] = L + n;
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

static int append_tokens(const char* fn, const void* x_bf16, const signed char* key_rows,
                         const long long* row_off, int* len, int B, int n, int n_layers,
                         long long layer_rows, int D, int Dk, unsigned char* kv_fp4,
                         unsigned char* kv_scale, signed char* keys, void* stream) {
    if (B < 0 || n < 0 || n_layers < 0 || layer_rows < 0)
        return fail(CSA2_ERR_INVALID, "%s: negative size", fn);
    if (B == 0 || n == 0) return CSA2_OK;
    if (!key_rows || !row_off || !len || !keys || (n_layers > 0 && (!x_bf16 || !kv_fp4 || !kv_scale)))
        return fail(CSA2_ERR_INVALID, "%s: null pointer", fn);
    if (Dk != kDk) return fail(CSA2_ERR_UNSUPPORTED, "%s: Dk must be 64", fn);
    if (D <= 0 || D % 32 != 0) return fail(CSA2_ERR_INVALID, "%s: D %% 32 != 0", fn);
    if (B > 65535) return fail(CSA2_ERR_UNSUPPORTED, "%s: B > 65535", fn);
    if ((long long)n * n_layers > (1ll << 30) || (long long)n * B > (1ll << 30))
        return fail(CSA2_ERR_UNSUPPORTED, "%s: n too large", fn);
    if (!aligned(x_bf16, 16) || !aligned(key_rows, 16) || !aligned(keys, 16) ||
        !aligned(kv_fp4, 4) || !aligned(row_off, 8) || !aligned(len, 4))
        return fail(CSA2_ERR_INVALID, "%s: misaligned pointer", fn);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const uint16_t* x16 = reinterpret_cast<const uint16_t*>(x_bf16);
    const long long items = (long long)n * n_layers;
    if (items <= 2 * kWideItems) {                    // one workgroup per sequence, one launch
        hipLaunchKernelGGL(append_token_kernel, dim3(B), dim3(kTokenThreads), 0, s, x16,
                           reinterpret_cast<const int8_t*>(key_rows), row_off, len, B, n,
                           n_layers, layer_rows, D, kv_fp4, kv_scale,
                           reinterpret_cast<int8_t*>(keys));
        return launch_status(fn);
    }
    const dim3 grid((unsigned)((items + kWideItems - 1) / kWideItems), (unsigned)B);
    hipLaunchKernelGGL(append_rows_wide_kernel, grid, dim3(kWideThreads), 0, s, x16, row_off, len,
                       B, n, n_layers, layer_rows, D, kv_fp4, kv_scale);
    if (int e = launch_status(fn)) return e;
    hipLaunchKernelGGL(append_keys_len_kernel, dim3(B), dim3(256), 0, s,
                       reinterpret_cast<const int8_t*>(key_rows), row_off, len, B, n,
                       reinterpret_cast<int8_t*>(keys));
    return launch_status(fn);
}

extern "C" int csa2_append_token(const void* x_bf16, const signed char* key_rows,
                                 const long long* row_off, int* len, int B, int n_layers,
                                 long long layer_rows, int D, int Dk, unsigned char* kv_fp4,
                                 unsigned char* kv_scale, signed char* keys, void* stream) {
    return append_tokens("csa2_append_token", x_bf16, key_rows, row_off, len, B, 1, n_layers,
                         layer_rows, D, Dk, kv_fp4, kv_scale, keys, stream);
}

extern "C" int csa2_append_tokens(const void* x_bf16, const signed char* key_rows,
                                  const long long* row_off, int* len, int B, int n, int n_layers,
                                  long long layer_rows, int D, int Dk, unsigned char* kv_fp4,
                                  unsigned char* kv_scale, signed char* keys, void* stream) {
    return append_tokens("csa2_append_tokens", x_bf16, key_rows, row_off, len, B, n, n_layers,
                         layer_rows, D, Dk, kv_fp4, kv_scale, keys, stream);
}
