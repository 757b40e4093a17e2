// csa2_select_topk: the k highest-ranked candidates of a scored list, ties
// to the lower position, output ascending ("How DeepSeek V4.1 Flash Actually
// Works", item 2: the 512 most relevant KV entries; "DeepSeek Has Done It
// Again...": up to 512 global positions).
//
// One workgroup (1,024 threads) per sequence.  The candidate scores (<= 16,384
// x 4 B) sit in LDS; an exact radix select over the 31-bit scores (digits of
// 11, 11 and 9 bits, LDS histograms, block-wide suffix scans) finds the
// threshold T and the number of ties to keep; an ordered compaction then
// writes s > T plus the first ties in list order.  Candidate lists are
// ascending in position, so list order is position order.
#include "abi_common.h"
#include "common.h"

namespace csa2 {

constexpr int kSelThreads = 1024;
constexpr int kSelMaxP = 16384;
constexpr int kSelWaves = kSelThreads / kWave;

// Exclusive prefix sum over the block (1,024 threads).
__device__ __forceinline__ int sel_block_scan(int v, int* s_tmp, int& total) {
    const int l = lane_id(), wv = threadIdx.x / kWave;
    int x = v;
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (l >= o) x += y;
    }
    if (l == kWave - 1) s_tmp[wv] = x;
    __syncthreads();
    int before = 0;
    total = 0;
    for (int i = 0; i < kSelWaves; ++i) {
        const int c = s_tmp[i];
        if (i < wv) before += c;
        total += c;
    }
    __syncthreads();
    return before + x - v;
}

__global__ __launch_bounds__(kSelThreads) void select_topk_kernel(
    const int* __restrict__ score, const int* __restrict__ cand_pos,
    const int* __restrict__ cand_len, int P, int k, int* __restrict__ sel_pos,
    int* __restrict__ sel_len) {
    __shared__ int s_sc[kSelMaxP];
    __shared__ uint32_t s_hist[2048];
    __shared__ int s_tmp[kSelWaves];
    __shared__ int s_res[2];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int n = max(0, min(cand_len[b], P));
    const int keff = min(k, n);
    const int* sc = score + (size_t)b * P;
    for (int i = tid; i < n; i += kSelThreads) s_sc[i] = sc[i];

    int prefix = 0;       // fixed high bits of the threshold
    int need = keff;      // entries still to take among those matching prefix
    const int shifts[3] = {20, 9, 0};
    const int widths[3] = {11, 11, 9};
    if (keff > 0) {
        for (int pass = 0; pass < 3; ++pass) {
            const int sh = shifts[pass], wd = widths[pass], nb = 1 << wd;
            for (int i = tid; i < nb; i += kSelThreads) s_hist[i] = 0;
            __syncthreads();
            const int hsh = sh + wd;
            for (int i = tid; i < n; i += kSelThreads) {
                const int s = s_sc[i];
                if ((s >> hsh) == (prefix >> hsh)) atomicAdd(&s_hist[(s >> sh) & (nb - 1)], 1u);
            }
            __syncthreads();
            // thread t owns bins 2r, 2r+1 with r = 1023 - t (high bins first)
            const int r = kSelThreads - 1 - tid;
            const int b0 = 2 * r, b1 = 2 * r + 1;
            const int c1 = b1 < nb ? (int)s_hist[b1] : 0;
            const int c0 = b0 < nb ? (int)s_hist[b0] : 0;
            int tot;
            const int above = sel_block_scan(c0 + c1, s_tmp, tot);
            if (above < need && need <= above + c0 + c1) {
                int d, a;
                if (need <= above + c1) {
                    d = b1;
                    a = above;
                } else {
                    d = b0;
                    a = above + c1;
                }
                s_res[0] = prefix | (d << sh);
                s_res[1] = need - a;
            }
            __syncthreads();
            prefix = s_res[0];
            need = s_res[1];
            __syncthreads();
        }
    }
    const int T = keff > 0 ? prefix : 0x7FFFFFFF;
    const int needT = keff > 0 ? need : 0;

    // ordered compaction, 16 contiguous entries per thread
    constexpr int PER = kSelMaxP / kSelThreads;
    const int i0 = tid * PER;
    int v[PER];
    int n_eq = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        v[j] = (i0 + j < n) ? s_sc[i0 + j] : -1;
        n_eq += (v[j] >= 0) & (v[j] == T);
    }
    int tot;
    int eq_rank = sel_block_scan(n_eq, s_tmp, tot);
    int n_sel = 0;
    uint32_t take = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        bool tk = false;
        if (v[j] < 0) tk = false;
        else if (v[j] > T) tk = true;
        else if (v[j] == T) {
            tk = eq_rank < needT;
            ++eq_rank;
        }
        take |= (uint32_t)tk << j;
        n_sel += tk;
    }
    int off = sel_block_scan(n_sel, s_tmp, tot);
    int* out = sel_pos + (size_t)b * k;
    const int* cp = cand_pos + (size_t)b * P;
#pragma unroll
    for (int j = 0; j < PER; ++j)
        if ((take & (1u << j)) && off < keff) out[off++] = cp[i0 + j];
    for (int i = keff + tid; i < k; i += kSelThreads) out[i] = -1;
    if (tid == 0) sel_len[b] = keff;
}

}  // namespace csa2

using namespace csa2;

extern "C" int csa2_select_topk(const int* score, const int* cand_pos, const int* cand_len, int B,
                                int P, int k, int* sel_pos, int* sel_len, void* ws,
                                size_t ws_bytes, void* stream) {
    (void)ws;
    (void)ws_bytes;
    if (B < 0) return fail(CSA2_ERR_INVALID, "csa2_select_topk: B < 0");
    if (B == 0) return CSA2_OK;
    if (!score || !cand_pos || !cand_len || !sel_pos || !sel_len)
        return fail(CSA2_ERR_INVALID, "csa2_select_topk: null pointer");
    if (k < 1 || k > P) return fail(CSA2_ERR_INVALID, "csa2_select_topk: need 1 <= k <= P");
    if (P > kSelMaxP) return fail(CSA2_ERR_UNSUPPORTED, "csa2_select_topk: P > %d", kSelMaxP);
    hipLaunchKernelGGL(select_topk_kernel, dim3(B), dim3(kSelThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), score, cand_pos, cand_len, P, k,
                       sel_pos, sel_len);
    return launch_status("csa2_select_topk launch");
}
