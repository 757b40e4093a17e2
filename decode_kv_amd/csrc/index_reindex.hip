// csa2_index_reindex: Reindex mode, re-scoring only the candidate pool with
// the layer's own index query ("DeepSeek V4.1-Flash 552B runs like 16B
// (CED)", "Act 2": later layers search only that much smaller pool; "How
// DeepSeek V4.1 Flash Actually Works", item 2: later layers search within the
// shortlist).
//
// Same int8 MFMA scoring as the Full scan, with the key operand gathered:
// each lane loads 16 bytes of the 64-byte key row of its candidate, four lanes
// per row, so every row costs one 64-byte segment.
#include "abi_common.h"
#include "common.h"

namespace csa2 {

constexpr int kReThreads = 256;  // 4 waves x 64 candidates

template <int NB>
__global__ __launch_bounds__(kReThreads) void reindex_kernel(
    const int8_t* __restrict__ q, const int8_t* __restrict__ wts,
    const int8_t* __restrict__ keys, const long long* __restrict__ row_off,
    const int* __restrict__ cand_pos, const int* __restrict__ cand_len, int H, int P,
    int* __restrict__ score) {
    const int b = blockIdx.y;
    const int l = lane_id();
    const int base = blockIdx.x * kReThreads + (threadIdx.x / kWave) * kWave;
    if (base >= P) return;
    const int* cp = cand_pos + (size_t)b * P;
    int* out = score + (size_t)b * P;
    // round trip 1: the list length, this wave's four groups of candidate
    // positions (indices clamped into the row, so every load is unconditional),
    // the index query and the row offset
    int pos[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) pos[u] = cp[min(base + 16 * u + (l & 15), P - 1)];
    const int n = min(cand_len[b], P);
    i32x4 qa[NB];
    uint32_t wr[NB][4];
    load_index_query<NB>(q + (size_t)b * H * kDk, wts + (size_t)b * H, H, qa, wr);
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
    const int mine = (int)reduce_rows4(part);          // candidate base + l
    const int i = base + l;
    if (i < P) out[i] = i < n ? mine : -1;
}

}  // namespace csa2

using namespace csa2;

extern "C" int csa2_index_reindex(const signed char* q, const signed char* w,
                                  const signed char* keys, const long long* row_off,
                                  const int* cand_pos, const int* cand_len, int B, int H,
                                  int Dk, int P, int* score, void* stream) {
    if (B < 0) return fail(CSA2_ERR_INVALID, "csa2_index_reindex: B < 0");
    if (B == 0) return CSA2_OK;
    if (!q || !w || !keys || !row_off || !cand_pos || !cand_len || !score)
        return fail(CSA2_ERR_INVALID, "csa2_index_reindex: null pointer");
    if (Dk != kDk) return fail(CSA2_ERR_UNSUPPORTED, "csa2_index_reindex: Dk must be 64");
    if (H < 1 || H > 64) return fail(CSA2_ERR_INVALID, "csa2_index_reindex: H must be in [1, 64]");
    if (P < 1) return fail(CSA2_ERR_INVALID, "csa2_index_reindex: P < 1");
    if (B > 65535) return fail(CSA2_ERR_UNSUPPORTED, "csa2_index_reindex: B > 65535");
    if (!aligned(q, 16) || !aligned(keys, 16) || !aligned(row_off, 8))
        return fail(CSA2_ERR_INVALID, "csa2_index_reindex: misaligned pointer");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const dim3 grid((P + kReThreads - 1) / kReThreads, B);
    const int8_t* q8 = reinterpret_cast<const int8_t*>(q);
    const int8_t* w8 = reinterpret_cast<const int8_t*>(w);
    const int8_t* k8 = reinterpret_cast<const int8_t*>(keys);
    switch ((H + 15) / 16) {
        case 1: hipLaunchKernelGGL(reindex_kernel<1>, grid, dim3(kReThreads), 0, s, q8, w8, k8, row_off, cand_pos, cand_len, H, P, score); break;
        case 2: hipLaunchKernelGGL(reindex_kernel<2>, grid, dim3(kReThreads), 0, s, q8, w8, k8, row_off, cand_pos, cand_len, H, P, score); break;
        case 3: hipLaunchKernelGGL(reindex_kernel<3>, grid, dim3(kReThreads), 0, s, q8, w8, k8, row_off, cand_pos, cand_len, H, P, score); break;
        default: hipLaunchKernelGGL(reindex_kernel<4>, grid, dim3(kReThreads), 0, s, q8, w8, k8, row_off, cand_pos, cand_len, H, P, score); break;
    }
    return launch_status("csa2_index_reindex launch");
}
