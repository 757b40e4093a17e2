// csa2_select_topk: the k highest-ranked candidates of a scored list, ties
// to the lower position, output ascending ("How DeepSeek V4.1 Flash Actually
// Works", item 2: the 512 most relevant KV entries; "DeepSeek Has Done It
// Again...": up to 512 global positions).
//
// One workgroup (1,024 threads) per sequence.  The candidate scores (<= 16,384
// x 4 B) are loaded with all of a thread's loads in flight and kept both in
// registers and in LDS.  An exact radix select finds the threshold T and the
// number of ties to keep: a first histogram over a float-like 12-bit key
// (exponent + 7 mantissa bits, so pool scores spread over many bins and the
// LDS atomics rarely collide), then 13-bit refinement digits inside the chosen
// bin until one value remains.  An ordered compaction writes s > T plus the
// first ties in list order.  Candidate lists are ascending in position, so
// list order is position order.
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

// Monotone 12-bit key of a non-negative score: exact below 128, otherwise the
// exponent and the 7 bits below the leading one.
__device__ __forceinline__ int sel_key(int s) {
    if (s < 128) return s;
    const int e = 31 - __clz(s);
    return ((e - 6) << 7) | ((s >> (e - 7)) & 127);    // < 25 * 128 = 3200
}

constexpr int kSelKeyBins = 3200;
constexpr int kSelRefBins = 8192;   // 13-bit refinement digit

// The bin holding the need-th largest entry of an LDS histogram (bins in
// ascending value order): writes (bin, entries in higher bins) to s_res.
__device__ __forceinline__ void sel_find_bin(const uint32_t* s_hist, int nb, int need,
                                             int* s_tmp, int* s_res) {
    const int per = (nb + kSelThreads - 1) / kSelThreads;
    const int r = kSelThreads - 1 - threadIdx.x;            // thread 0 owns the top bins
    int mysum = 0;
    for (int i = 0; i < per; ++i) {
        const int bin = r * per + i;
        mysum += bin < nb ? (int)s_hist[bin] : 0;
    }
    int tot;
    const int above = sel_block_scan(mysum, s_tmp, tot);
    if (above < need && need <= above + mysum) {
        int acc = above;
        for (int i = per - 1; i >= 0; --i) {
            const int bin = r * per + i;
            const int c = bin < nb ? (int)s_hist[bin] : 0;
            if (acc + c >= need) {
                s_res[0] = bin;
                s_res[1] = acc;
                break;
            }
            acc += c;
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(kSelThreads) void select_topk_kernel(
    const int* __restrict__ score, const int* __restrict__ cand_pos,
    const int* __restrict__ cand_len, int P, int k, int* __restrict__ sel_pos,
    int* __restrict__ sel_len) {
    __shared__ int s_sc[kSelMaxP];
    __shared__ uint32_t s_hist[kSelRefBins];
    __shared__ int s_tmp[kSelWaves];
    __shared__ int s_res[2];
    __shared__ int s_cs[kSelThreads], s_ci[kSelThreads];   // threshold-bin entries
    constexpr int PER = kSelMaxP / kSelThreads;   // 16
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int n = max(0, min(cand_len[b], P));
    const int keff = min(k, n);
    const int* sc = score + (size_t)b * P;

    // all 16 loads of a thread in flight at once; strided for coalescing
    int v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int i = tid + j * kSelThreads;
        v[j] = i < n ? sc[i] : -1;          // valid scores are >= 0
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) s_sc[tid + j * kSelThreads] = v[j];

    int T = 0x7FFFFFFF, needT = 0;
    if (keff > 0) {
        // pass 0: float-like key, fine enough that the atomics rarely collide
        for (int i = tid; i < kSelKeyBins; i += kSelThreads) s_hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < PER; ++j)
            if (v[j] >= 0) atomicAdd(&s_hist[sel_key(v[j])], 1u);
        __syncthreads();
        sel_find_bin(s_hist, kSelKeyBins, keff, s_tmp, s_res);
        const int kb = s_res[0];
        int need = keff - s_res[1];
        const int m = (int)s_hist[kb];        // entries inside the threshold bin
        int lo, hi;
        if (kb < 128) {
            lo = hi = kb;
        } else {
            const int e = (kb >> 7) + 6;
            lo = (128 + (kb & 127)) << (e - 7);
            hi = lo + (1 << (e - 7)) - 1;
        }
        if (m <= kSelThreads) {
            // few entries in the bin: rank them exactly by (score desc, index asc)
            int cnt = 0;
#pragma unroll
            for (int j = 0; j < PER; ++j) cnt += v[j] >= lo && v[j] <= hi;
            int tot;
            int o = sel_block_scan(cnt, s_tmp, tot);
#pragma unroll
            for (int j = 0; j < PER; ++j)
                if (v[j] >= lo && v[j] <= hi) {
                    s_cs[o] = v[j];
                    s_ci[o] = tid + j * kSelThreads;
                    ++o;
                }
            __syncthreads();
            if (tid < m) {
                const int cs = s_cs[tid], ci = s_ci[tid];
                int gt = 0, eq_lower = 0;
                for (int u = 0; u < m; ++u) {
                    const int us = s_cs[u];
                    gt += us > cs;
                    eq_lower += (us == cs) & (s_ci[u] < ci);
                }
                if (gt + eq_lower == need - 1) {   // exactly one entry has this rank
                    s_res[0] = cs;
                    s_res[1] = eq_lower + 1;
                }
            }
            __syncthreads();
            T = s_res[0];
            needT = s_res[1];
        } else {
            // many entries: 13-bit refinement passes inside [lo, hi]
            while (lo < hi) {
                const unsigned width = (unsigned)(hi - lo) + 1u;
                const int bits = 32 - __clz(width - 1u);
                const int sh = bits > 13 ? bits - 13 : 0;
                const int nb = (int)(((width - 1u) >> sh) + 1u);
                __syncthreads();
                for (int i = tid; i < nb; i += kSelThreads) s_hist[i] = 0;
                __syncthreads();
#pragma unroll
                for (int j = 0; j < PER; ++j)
                    if (v[j] >= lo && v[j] <= hi) atomicAdd(&s_hist[(v[j] - lo) >> sh], 1u);
                __syncthreads();
                sel_find_bin(s_hist, nb, need, s_tmp, s_res);
                const int d = s_res[0];
                need -= s_res[1];
                const int nlo = lo + (d << sh);
                const int nhi = (sh == 0) ? nlo : min(hi, nlo + (1 << sh) - 1);
                lo = nlo;
                hi = nhi;
            }
            T = lo;
            needT = need;
        }
    }
    __syncthreads();

    // ordered compaction: thread t owns entries [16t, 16t + 16)
    const int i0 = tid * PER;
    int w[PER];
    int n_eq = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        w[j] = s_sc[i0 + j];
        n_eq += (w[j] >= 0) & (w[j] == T);
    }
    int tot;
    int eq_rank = sel_block_scan(n_eq, s_tmp, tot);
    int n_sel = 0;
    uint32_t take = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        bool tk = false;
        if (w[j] < 0) tk = false;
        else if (w[j] > T) tk = true;
        else if (w[j] == T) {
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
