// csa2_index_reindex: Reindex mode, re-scoring only the candidate pool with
// the layer's own index query.  ("DeepSeek V4.1-Flash 552B runs like 16B
// (CED)", "Act 2", and "How DeepSeek V4.1 Flash Actually Works", item 2: a
// Reindex layer ranks the Full layer's pool again instead of the context.)
//
// Same int8 MFMA scoring as the Full scan, with the key operand gathered:
// each lane loads 16 bytes of the 64-byte key row of its candidate, four lanes
// per row, so every row costs one 64-byte segment.
#include <type_traits>

#include "abi_common.h"
#include "common.h"

namespace csa2 {

constexpr int kReThreads = 256;  // 4 waves x 64 candidates
constexpr int kSimds = 1024;     // 256 compute units x 4 SIMDs

// List y of a verify block of T tokens per sequence: shared (one list per
// sequence, scored with the best score over the block's tokens) or per token
// (list y = b * T + t, scored with token t's query).  T == 1 is the plain
// one-token step, whose instance (BLOCK false) carries none of the block's
// bookkeeping.
template <int NB, bool BLOCK>
__global__ __launch_bounds__(kReThreads) void reindex_kernel(
    const int8_t* __restrict__ q, const int8_t* __restrict__ wts,
    const int8_t* __restrict__ keys, const long long* __restrict__ row_off,
    const int* __restrict__ cand_pos, const int* __restrict__ cand_len, int H, int P,
    int* __restrict__ score, int T, int shared) {
    const int y = blockIdx.y;
    const int b = BLOCK && !shared ? y / T : y;          // sequence: its keys
    const int tk0 = BLOCK && !shared ? y - b * T : 0;    // tokens tk0 .. tk1 - 1 score the list
    const int tk1 = !BLOCK ? 1 : (shared ? T : tk0 + 1);
    const int l = lane_id();
    const int base = blockIdx.x * kReThreads + (threadIdx.x / kWave) * kWave;
    if (base >= P) return;
    const int* cp = cand_pos + (size_t)y * P;
    int* out = score + (size_t)y * P;
    // round trip 1: the list length, this wave's four groups of candidate
    // positions (indices clamped into the row, so every load is unconditional),
    // the index query and the row offset
    int pos[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) pos[u] = cp[min(base + 16 * u + (l & 15), P - 1)];
    const int n = min(cand_len[y], P);
    i32x4 qa[NB];
    uint32_t wr[NB][4];
    const size_t qrow = BLOCK ? (size_t)b * T + tk0 : (size_t)b;   // the first token's query
    load_index_query<NB>(q + qrow * H * kDk, wts + qrow * H, H, qa, wr);
    const long long roff = row_off[b];
    if (base >= n) {
        if (base + l < P) out[base + l] = -1;
        return;
    }
    // round trip 2: every group's key rows (entries past the list read the
    // sequence's first candidate row, which exists since n > 0)
    const int8_t* kb = keys + (size_t)roff * kDk + (l >> 4) * 16;
    const int pos0 = __builtin_amdgcn_readfirstlane(pos[0]);   // lane 0 of group 0: entry base < n
    i32x4 kop[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int i = base + 16 * u + (l & 15);
        const int p = (i < n && pos[u] >= 0) ? pos[u] : pos0;
        kop[u] = *reinterpret_cast<const i32x4*>(kb + (size_t)p * kDk);
    }
    uint32_t part[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) part[u] = score_partial16<NB>(qa, wr, kop[u]);
    int mine = (int)reduce_rows4(part);                // candidate base + l
    if constexpr (BLOCK) {
        for (int tk = tk0 + 1; tk < tk1; ++tk) {         // shared list: best over the block
            const size_t r = (size_t)b * T + tk;
            load_index_query<NB>(q + r * H * kDk, wts + r * H, H, qa, wr);
#pragma unroll
            for (int u = 0; u < 4; ++u) part[u] = score_partial16<NB>(qa, wr, kop[u]);
            mine = max(mine, (int)reduce_rows4(part));
        }
    }
    const int i = base + l;
    if (i < P) out[i] = i < n ? mine : -1;
}

// A shared list of a block of T > 1 tokens when the lists are few: the
// workgroup's four waves score the same 64 candidates, wave w with tokens
// w, w + 4, ..., and the best score over the block goes through LDS (each
// wave's chain is about a quarter of one wave scoring every token).
template <int NB>
__global__ __launch_bounds__(kReThreads) void reindex_shared_kernel(
    const int8_t* __restrict__ q, const int8_t* __restrict__ wts,
    const int8_t* __restrict__ keys, const long long* __restrict__ row_off,
    const int* __restrict__ cand_pos, const int* __restrict__ cand_len, int H, int P,
    int* __restrict__ score, int T) {
    constexpr int NW = kReThreads / kWave;
    __shared__ int s_best[NW][kWave];
    const int b = blockIdx.y;
    const int l = lane_id(), wave = threadIdx.x / kWave;
    const int base = blockIdx.x * kWave;                 // this workgroup's 64 candidates
    if (base >= P) return;                               // uniform
    const int* cp = cand_pos + (size_t)b * P;
    int* out = score + (size_t)b * P;
    int pos[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) pos[u] = cp[min(base + 16 * u + (l & 15), P - 1)];
    const int n = min(cand_len[b], P);
    i32x4 qa[NB];
    uint32_t wr[NB][4];
    const bool has = wave < T;                           // uniform per wave
    if (has) load_index_query<NB>(q + ((size_t)b * T + wave) * H * kDk,
                                  wts + ((size_t)b * T + wave) * H, H, qa, wr);
    const long long roff = row_off[b];
    if (base >= n) {                                     // uniform
        if (wave == 0 && base + l < P) out[base + l] = -1;
        return;
    }
    int mine = -1;                                       // below every valid score
    if (has) {
        const int8_t* kb = keys + (size_t)roff * kDk + (l >> 4) * 16;
        const int pos0 = __builtin_amdgcn_readfirstlane(pos[0]);
        i32x4 kop[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = base + 16 * u + (l & 15);
            const int p = (i < n && pos[u] >= 0) ? pos[u] : pos0;
            kop[u] = *reinterpret_cast<const i32x4*>(kb + (size_t)p * kDk);
        }
        for (int tk = wave; tk < T; tk += NW) {
            if (tk != wave) {
                const size_t r = (size_t)b * T + tk;
                load_index_query<NB>(q + r * H * kDk, wts + r * H, H, qa, wr);
            }
            uint32_t part[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) part[u] = score_partial16<NB>(qa, wr, kop[u]);
            const int sc = (int)reduce_rows4(part);      // candidate base + l
            mine = tk == wave ? sc : max(mine, sc);
        }
    }
    s_best[wave][l] = mine;
    __syncthreads();
    if (wave == 0) {
        int best = s_best[0][l];
#pragma unroll
        for (int v = 1; v < NW; ++v)
            if (v < T) best = max(best, s_best[v][l]);
        const int i = base + l;
        if (i < P) out[i] = i < n ? best : -1;
    }
}

static int reindex(const char* fn, const signed char* q, const signed char* w,
                   const signed char* keys, const long long* row_off, const int* cand_pos,
                   const int* cand_len, int B, int T, int shared, int H, int Dk, int P,
                   int* score, void* stream) {
    if (B < 0) return fail(CSA2_ERR_INVALID, "%s: B < 0", fn);
    if (T < 1 || shared < 0 || shared > 1)
        return fail(CSA2_ERR_INVALID, "%s: T < 1 or shared not 0/1", fn);
    if (B == 0) return CSA2_OK;
    if (!q || !w || !keys || !row_off || !cand_pos || !cand_len || !score)
        return fail(CSA2_ERR_INVALID, "%s: null pointer", fn);
    if (Dk != kDk) return fail(CSA2_ERR_UNSUPPORTED, "%s: Dk must be 64", fn);
    if (H < 1 || H > 64) return fail(CSA2_ERR_INVALID, "%s: H must be in [1, 64]", fn);
    if (P < 1) return fail(CSA2_ERR_INVALID, "%s: P < 1", fn);
    const long long lists = shared ? (long long)B : (long long)B * T;
    if (lists > 65535) return fail(CSA2_ERR_UNSUPPORTED, "%s: more than 65535 lists", fn);
    if (!aligned(q, 16) || !aligned(keys, 16) || !aligned(row_off, 8))
        return fail(CSA2_ERR_INVALID, "%s: misaligned pointer", fn);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const dim3 grid((P + kReThreads - 1) / kReThreads, (unsigned)lists);
    const int8_t* q8 = reinterpret_cast<const int8_t*>(q);
    const int8_t* w8 = reinterpret_cast<const int8_t*>(w);
    const int8_t* k8 = reinterpret_cast<const int8_t*>(keys);
    // shared lists and too few plain waves to give every SIMD one (measured:
    // one 1M sequence's five-token block scores 27% faster split, a batch of
    // eight 15% slower, its extra key gathers outweighing the shorter chains)
    const long long plain_waves = (long long)lists * ((P + kWave - 1) / kWave);
    if (shared && T > 1 && plain_waves < kSimds) {
        const dim3 g2((P + kWave - 1) / kWave, (unsigned)lists);
        switch ((H + 15) / 16) {
            case 1: hipLaunchKernelGGL(reindex_shared_kernel<1>, g2, dim3(kReThreads), 0, s, q8, w8, k8, row_off, cand_pos, cand_len, H, P, score, T); break;
            case 2: hipLaunchKernelGGL(reindex_shared_kernel<2>, g2, dim3(kReThreads), 0, s, q8, w8, k8, row_off, cand_pos, cand_len, H, P, score, T); break;
            case 3: hipLaunchKernelGGL(reindex_shared_kernel<3>, g2, dim3(kReThreads), 0, s, q8, w8, k8, row_off, cand_pos, cand_len, H, P, score, T); break;
            default: hipLaunchKernelGGL(reindex_shared_kernel<4>, g2, dim3(kReThreads), 0, s, q8, w8, k8, row_off, cand_pos, cand_len, H, P, score, T); break;
        }
        return launch_status(fn);
    }
    auto launch = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, grid, dim3(kReThreads), 0, s, q8, w8, k8, row_off, cand_pos,
                           cand_len, H, P, score, T, shared);
    };
    auto launch_nb = [&](auto blk) {
        constexpr bool BLK = decltype(blk)::value;
        switch ((H + 15) / 16) {
            case 1: launch(reindex_kernel<1, BLK>); break;
            case 2: launch(reindex_kernel<2, BLK>); break;
            case 3: launch(reindex_kernel<3, BLK>); break;
            default: launch(reindex_kernel<4, BLK>); break;
        }
    };
    if (T > 1)
        launch_nb(std::true_type{});
    else
        launch_nb(std::false_type{});
    return launch_status(fn);
}

}  // namespace csa2

using namespace csa2;

extern "C" int csa2_index_reindex(const signed char* q, const signed char* w,
                                  const signed char* keys, const long long* row_off,
                                  const int* cand_pos, const int* cand_len, int B, int H,
                                  int Dk, int P, int* score, void* stream) {
    return reindex("csa2_index_reindex", q, w, keys, row_off, cand_pos, cand_len, B, 1, 0, H, Dk,
                   P, score, stream);
}

extern "C" int csa2_index_reindex_block(const signed char* q, const signed char* w,
                                        const signed char* keys, const long long* row_off,
                                        const int* cand_pos, const int* cand_len, int B, int T,
                                        int shared, int H, int Dk, int P, int* score,
                                        void* stream) {
    return reindex("csa2_index_reindex_block", q, w, keys, row_off, cand_pos, cand_len, B, T,
                   shared, H, Dk, P, score, stream);
}
