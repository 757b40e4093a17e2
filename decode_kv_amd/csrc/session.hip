// csa2_session_export / csa2_session_import: the part of a sequence's cache
// state that outlives a session, and its restore.
// ("How DeepSeek V4.1 Flash Actually Works", "The three KV-cache
// optimizations", item 3: the local state of the newest 128 tokens is kept
// only while a session is active and is rebuilt later by replaying those
// tokens; "DeepSeek V4.1-Flash 552B runs like 16B (CED)", "Act 3: FP4 KV & SWA
// Bounded Replay": recomputing the recent tokens replaces storing them.)
//
// A sequence of length L keeps positions [0, L - R) (R = the replay window,
// at most L): their index keys and the FP4 codes and scales of every layer.
// The newest R positions are dropped; after an import their rows come back
// by appending the replayed tokens (csa2_append_tokens).
//
// One copy kernel for both directions: workgroup (x, b) moves positions
// [64 x, 64 x + 64) of sequence b, 16 bytes per thread and step, between the
// caches (rows row_off[b] + p, layer l at l * layer_rows) and the compact
// saved arrays ([B][cap] rows per layer).
#include "abi_common.h"
#include "common.h"

namespace csa2 {

constexpr int kSessThreads = 256;
constexpr int kSessRows = 64;    // positions per workgroup

struct SessArgs {
    const long long* row_off;
    int* len;                    // import: set to the saved length
    const int* saved_len;        // import: saved positions per sequence
    int* out_len;                // export: saved positions per sequence
    int B, replay, n_layers, D;
    long long cap, layer_rows;
    unsigned char* kv_fp4;
    unsigned char* kv_scale;
    signed char* keys;
    unsigned char* s_fp4;        // [n_layers][B][cap][D/2]
    unsigned char* s_scale;      // [n_layers][B][cap][D/32]
    signed char* s_keys;         // [B][cap][Dk]
};

template <bool EXPORT>
__global__ __launch_bounds__(kSessThreads) void session_copy_kernel(SessArgs a) {
    const int b = blockIdx.y;
    int n;                                            // positions kept for sequence b
    if (EXPORT) {
        const int L = a.len[b];
        n = (int)min((long long)max(0, L - min(a.replay, max(L, 0))), a.cap);
        if (blockIdx.x == 0 && threadIdx.x == 0) a.out_len[b] = n;
    } else {
        n = (int)min((long long)max(0, a.saved_len[b]), a.cap);
        if (blockIdx.x == 0 && threadIdx.x == 0) a.len[b] = n;
    }
    const long long p0 = (long long)blockIdx.x * kSessRows;
    if (p0 >= n) return;
    const int np = (int)min((long long)kSessRows, n - p0);
    const long long roff = a.row_off[b];
    const int F = a.D / 32;                           // 16-byte pieces of a code row
    const int S = a.D / 512;                          // 16-byte pieces of a scale row
    const int per_pos = kDk / 16 + a.n_layers * (F + S);
    const long long total = (long long)np * per_pos;
    for (long long c = threadIdx.x; c < total; c += kSessThreads) {
        const int pi = (int)(c / per_pos);
        int f = (int)(c - (long long)pi * per_pos);
        const long long p = p0 + pi;                  // position
        const long long crow = roff + p;              // its cache row (layer 0)
        const long long srow = (long long)b * a.cap + p;   // its saved row
        u32x4* dst;
        const u32x4* src;
        if (f < kDk / 16) {
            u32x4* kc = reinterpret_cast<u32x4*>(a.keys + crow * kDk) + f;
            u32x4* ks = reinterpret_cast<u32x4*>(a.s_keys + srow * kDk) + f;
            dst = EXPORT ? ks : kc;
            src = EXPORT ? kc : ks;
        } else {
            f -= kDk / 16;
            const int layer = f / (F + S);
            f -= layer * (F + S);
            const long long cl = layer * a.layer_rows + crow;
            const long long sl = (long long)layer * a.B * a.cap + srow;
            u32x4 *cc, *sc;
            if (f < F) {
                cc = reinterpret_cast<u32x4*>(a.kv_fp4 + cl * (a.D / 2)) + f;
                sc = reinterpret_cast<u32x4*>(a.s_fp4 + sl * (a.D / 2)) + f;
            } else {
                cc = reinterpret_cast<u32x4*>(a.kv_scale + cl * (a.D / 32)) + (f - F);
                sc = reinterpret_cast<u32x4*>(a.s_scale + sl * (a.D / 32)) + (f - F);
            }
            dst = EXPORT ? sc : cc;
            src = EXPORT ? cc : sc;
        }
        *dst = *src;
    }
}

static int session_check(const char* fn, const SessArgs& a, int Dk) {
    if (a.B < 0 || a.cap < 0 || a.n_layers < 0 || a.layer_rows < 0 || a.replay < 0)
        return fail(CSA2_ERR_INVALID, "%s: negative size", fn);
    if (a.B == 0) return CSA2_OK;
    if (!a.row_off || !a.len || !a.keys || !a.s_keys ||
        (a.n_layers > 0 && (!a.kv_fp4 || !a.kv_scale || !a.s_fp4 || !a.s_scale)))
        return fail(CSA2_ERR_INVALID, "%s: null pointer", fn);
    if (Dk != kDk) return fail(CSA2_ERR_UNSUPPORTED, "%s: Dk must be 64", fn);
    if (a.D <= 0 || a.D % 512 != 0) return fail(CSA2_ERR_UNSUPPORTED, "%s: D must be a multiple of 512", fn);
    if (a.B > 65535) return fail(CSA2_ERR_UNSUPPORTED, "%s: B > 65535", fn);
    if ((a.cap + kSessRows - 1) / kSessRows > 0x7FFFFFFFll)
        return fail(CSA2_ERR_UNSUPPORTED, "%s: cap too large", fn);
    const void* ptrs[] = {a.kv_fp4, a.kv_scale, a.keys, a.s_fp4, a.s_scale, a.s_keys};
    for (const void* p : ptrs)
        if (!aligned(p, 16)) return fail(CSA2_ERR_INVALID, "%s: misaligned pointer", fn);
    if (!aligned(a.row_off, 8) || !aligned(a.len, 4))
        return fail(CSA2_ERR_INVALID, "%s: misaligned pointer", fn);
    return CSA2_OK;
}

static int session_launch(bool exp, const SessArgs& a, void* stream, const char* fn) {
    const long long gx = (a.cap + kSessRows - 1) / kSessRows;
    if (gx == 0) return CSA2_OK;
    const dim3 grid((unsigned)gx, (unsigned)a.B);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (exp)
        hipLaunchKernelGGL(session_copy_kernel<true>, grid, dim3(kSessThreads), 0, s, a);
    else
        hipLaunchKernelGGL(session_copy_kernel<false>, grid, dim3(kSessThreads), 0, s, a);
    return launch_status(fn);
}

}  // namespace csa2

using namespace csa2;

extern "C" int csa2_session_export(const long long* row_off, const int* len, int B, int replay,
                                   long long cap, int n_layers, long long layer_rows, int D,
                                   int Dk, const unsigned char* kv_fp4,
                                   const unsigned char* kv_scale, const signed char* keys,
                                   unsigned char* saved_fp4, unsigned char* saved_scale,
                                   signed char* saved_keys, int* saved_len, void* stream) {
    const char* fn = "csa2_session_export";
    SessArgs a = {};
    a.row_off = row_off;
    a.len = const_cast<int*>(len);          // read only in this direction
    a.out_len = saved_len;
    a.B = B;
    a.replay = replay;
    a.n_layers = n_layers;
    a.D = D;
    a.cap = cap;
    a.layer_rows = layer_rows;
    a.kv_fp4 = const_cast<unsigned char*>(kv_fp4);
    a.kv_scale = const_cast<unsigned char*>(kv_scale);
    a.keys = const_cast<signed char*>(keys);
    a.s_fp4 = saved_fp4;
    a.s_scale = saved_scale;
    a.s_keys = saved_keys;
    if (int e = session_check(fn, a, Dk)) return e;
    if (B == 0) return CSA2_OK;
    if (!saved_len || !aligned(saved_len, 4)) return fail(CSA2_ERR_INVALID, "%s: saved_len", fn);
    return session_launch(true, a, stream, fn);
}

extern "C" int csa2_session_import(const long long* row_off, int* len, const int* saved_len,
                                   int B, long long cap, int n_layers, long long layer_rows,
                                   int D, int Dk, const unsigned char* saved_fp4,
                                   const unsigned char* saved_scale, const signed char* saved_keys,
                                   unsigned char* kv_fp4, unsigned char* kv_scale,
                                   signed char* keys, void* stream) {
    const char* fn = "csa2_session_import";
    SessArgs a = {};
    a.row_off = row_off;
    a.len = len;
    a.saved_len = saved_len;
    a.B = B;
    a.n_layers = n_layers;
    a.D = D;
    a.cap = cap;
    a.layer_rows = layer_rows;
    a.kv_fp4 = kv_fp4;
    a.kv_scale = kv_scale;
    a.keys = keys;
    a.s_fp4 = const_cast<unsigned char*>(saved_fp4);
    a.s_scale = const_cast<unsigned char*>(saved_scale);
    a.s_keys = const_cast<signed char*>(saved_keys);
    if (int e = session_check(fn, a, Dk)) return e;
    if (B == 0) return CSA2_OK;
    if (!saved_len || !aligned(saved_len, 4)) return fail(CSA2_ERR_INVALID, "%s: saved_len", fn);
    return session_launch(false, a, stream, fn);
}
