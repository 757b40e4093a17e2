// csa2_select_topk: the k highest-ranked candidates of a scored list, ties
// to the lower position, output ascending.  ("How DeepSeek V4.1 Flash Actually
// Works", item 2, and "DeepSeek Has Done It Again...", "Architecture and
// inference efficiency": each layer attends to a selection of 512 positions
// from the history.)
//
// One workgroup (1,024 threads) per sequence.  The candidate scores and
// positions (<= 16,384 each) are loaded with all of a thread's loads in
// flight and kept in registers (entry i lives in thread i mod 1,024).  An
// exact radix select finds the threshold T and the number of ties at T to
// keep: a first histogram over a float-like 12-bit key (exponent + 7
// mantissa bits, so pool scores spread over many bins and the LDS atomics
// rarely collide) picks the bin holding the k-th largest score; further
// digits inside that bin narrow it to the single value T.  The output is an
// ordered compaction of s > T plus the first ties in list order; candidate
// lists are ascending in position, so list order is position order.
//
// Usually the chosen bin and the bins above it hold at most 1,024 entries:
// they are then compacted to LDS once, in list order, one per thread, and
// 8-bit digit passes, the tie order and the output all run on that set
// instead of on all 16 entries of every thread.  Lists with more entries
// there (heavy ties, k near P) take the general path: 13-bit digit passes
// over every entry until the bin holds at most 1,024, which are gathered one
// per thread for the last digits, then ballot-and-prefix compactions over
// all entries for the tie order and the output.
#include "abi_common.h"
#include "common.h"

namespace csa2 {

constexpr int kSelThreads = 1024;
constexpr int kSelMaxP = 16384;
constexpr int kSelWaves = kSelThreads / kWave;

// Monotone 12-bit key of a non-negative score: exact below 128, otherwise the
// exponent and the 7 bits below the leading one.  With sh = max(e - 7, 0) for
// the leading-one position e, s >> sh is the 8 leading bits (or s itself) and
// sh << 7 counts the octaves above 128, so the key is their sum (< 3200).
__device__ __forceinline__ int sel_key(int s) {
    const int sh = max(24 - (int)__builtin_clz((unsigned)s | 1u), 0);
    return (s >> sh) + (sh << 7);
}

constexpr int kSelKeyBins = 3200;
constexpr int kSelRefBins = 8192;   // 13-bit refinement digit
constexpr int kSelLast = kSelThreads;   // entries the last digits take, one per thread

// The bin holding the need-th largest entry of an LDS histogram (bins in
// ascending value order): writes (bin, entries in higher bins) to s_res.
__device__ __forceinline__ void sel_find_bin(const uint32_t* s_hist, int nb, int need,
                                             int* s_tmp, int* s_res) {
    const int per = (nb + kSelThreads - 1) / kSelThreads;
    const int r = kSelThreads - 1 - threadIdx.x;            // thread 0 owns the top bins
    // four bins per thread (the first pass): one 16-byte read each, so the
    // lanes of a wave read consecutive words instead of every fourth word
    // (a four-way LDS bank conflict); at most bin 4095 of the 8,192 is read
    u32x4 h4 = {0u, 0u, 0u, 0u};
    if (per == 4) h4 = *reinterpret_cast<const u32x4*>(s_hist + 4 * r);
    int mysum = 0;
    for (int i = 0; i < per; ++i) {
        const int bin = r * per + i;
        mysum += bin < nb ? (int)(per == 4 ? h4[i & 3] : s_hist[bin]) : 0;
    }
    int tot;
    const int above = block_exclusive_scan<kSelThreads>(mysum, s_tmp, tot);
    if (above < need && need <= above + mysum) {
        int acc = above;
        for (int i = per - 1; i >= 0; --i) {
            const int bin = r * per + i;
            const int c = bin < nb ? (int)(per == 4 ? h4[i & 3] : s_hist[bin]) : 0;
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

// Exclusive prefix, in (slot j, wave) order, of per-(j, wave) counts in
// s_cnt[j * kSelWaves + wave]; result in s_pre[wave * 16 + j], so that each
// wave reads its 16 prefixes as four 16-byte loads (wave_prefixes).  Wave 0
// scans 4 entries per lane.
__device__ __forceinline__ void slot_wave_scan(const int* s_cnt, int* s_pre) {
    __syncthreads();
    if (threadIdx.x < kWave) {
        const int l = threadIdx.x;
        int c[4], sum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            c[i] = s_cnt[4 * l + i];
            sum += c[i];
        }
        int run = wave_inclusive_scan(sum) - sum;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int flat = 4 * l + i;                      // j * kSelWaves + wave
            s_pre[(flat % kSelWaves) * 16 + flat / kSelWaves] = run;
            run += c[i];
        }
    }
    __syncthreads();
}

// This wave's 16 slot prefixes, all read before any is used.
__device__ __forceinline__ void wave_prefixes(const int* s_pre, int (&base)[16]) {
    const int4* p = reinterpret_cast<const int4*>(s_pre + (threadIdx.x / kWave) * 16);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int4 x = p[q];
        base[4 * q] = x.x;
        base[4 * q + 1] = x.y;
        base[4 * q + 2] = x.z;
        base[4 * q + 3] = x.w;
    }
}

// The usual case: the bin holding the keff-th largest score and the bins above
// it hold at most one entry per thread.  One ordered compaction moves those
// entries (in list order, which is position order) to LDS, one per thread,
// and the threshold, the ties and the output are found among them; no later
// pass touches the other entries.
//   v, pos: this thread's 16 entries (i = tid + 1024 j), invalid ones -1;
//   [lo, hi]: value range of that bin, cnt entries in it, need of them taken;
//   M: entries in the bin or above it (<= 1,024).
__device__ __forceinline__ void select_compacted(const int (&v)[kSelMaxP / kSelThreads],
                                                 const int (&pos)[kSelMaxP / kSelThreads], int lo,
                                                 int hi, int cnt, int need, int keff, int M, int k,
                                                 int* __restrict__ out, int* __restrict__ out_len,
                                                 uint32_t* s_hist, int* s_tmp, int* s_res,
                                                 int* s_cnt, int* s_pre, int* s_cs, int* s_cp) {
    constexpr int PER = kSelMaxP / kSelThreads;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    // ordered compaction: slot = rank of (j, wave, lane) among the entries >= lo
    // (branch-free: the 16 waves' exec-mask branches would share one scalar
    // unit; lane j stores slot j's count, unselected entries write to a spare
    // slot of their lane)
    uint64_t mi[PER];
    int my_cnt = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        mi[j] = __ballot(v[j] >= lo);                    // lo >= 0 excludes invalid entries
        my_cnt = lane == j ? (int)__popcll(mi[j]) : my_cnt;
    }
    if (lane < PER) s_cnt[lane * kSelWaves + wave] = my_cnt;
    slot_wave_scan(s_cnt, s_pre);
    int base[PER];
    wave_prefixes(s_pre, base);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const bool sel = (mi[j] >> lane) & 1ull;
        const int slot = sel ? base[j] + lane_rank64(mi[j]) : kSelThreads + lane;
        s_cs[slot] = v[j];
        s_cp[slot] = pos[j];
    }
    __syncthreads();
    const int sv = tid < M ? s_cs[tid] : -1;             // this thread's compacted entry
    narrow_to_value(sv, lo, hi, need, cnt, s_hist, s_res);
    const int T = lo, needT = need;
    // take s > T, plus the first needT entries with s == T in position order:
    // one scan of (count above T) << 16 | (count at T) gives both prefixes
    // (each total <= 1,024), and the output slot is the entries taken before
    const bool gt = tid < M && sv > T;
    const bool eq = tid < M && sv == T;
    int tot;
    const int pre = block_exclusive_scan<kSelThreads>(gt ? 1 << 16 : (eq ? 1 : 0), s_tmp, tot);
    const int eq_before = pre & 0xFFFF;
    const bool take = gt || (eq && eq_before < needT);
    const int o = (pre >> 16) + min(eq_before, needT);
    if (take && o < keff) out[o] = s_cp[tid];
    for (int i = keff + tid; i < k; i += kSelThreads) out[i] = -1;
    if (tid == 0) *out_len = keff;
}

__global__ __launch_bounds__(kSelThreads) void select_topk_kernel(
    const int* __restrict__ score, const int* __restrict__ cand_pos,
    const int* __restrict__ cand_len, int P, int k, int* __restrict__ sel_pos,
    int* __restrict__ sel_len) {
    constexpr int PER = kSelMaxP / kSelThreads;   // 16
    static_assert(PER * kSelWaves == 4 * kWave, "slot_wave_scan covers 256 entries");
    __shared__ __attribute__((aligned(16))) uint32_t s_hist[kSelRefBins];
    __shared__ int s_tmp[kSelWaves];
    __shared__ int s_res[4];
    static_assert(PER == 16 && kSelWaves == 16, "slot prefixes are 16 x 16");
    __shared__ int s_cnt[PER * kSelWaves];
    __shared__ __attribute__((aligned(16))) int s_pre[PER * kSelWaves];
    // compacted scores and positions, plus one spare slot per lane
    __shared__ int s_cs[kSelThreads + kWave], s_cp[kSelThreads + kWave];
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int* sc = score + (size_t)b * P;
    const int* cp = cand_pos + (size_t)b * P;
    // entry i = tid + 1024 j: every score of the row is loaded without waiting
    // for the list length (one memory round trip for both); positions follow
    const int len_b = cand_len[b];
    int v[PER], pos[PER];
    // (indices past P reread entry P - 1; they are past n and masked below)
#pragma unroll
    for (int j = 0; j < PER; ++j) v[j] = sc[min(tid + j * kSelThreads, P - 1)];
#pragma unroll
    for (int j = 0; j < PER; ++j) pos[j] = cp[min(tid + j * kSelThreads, P - 1)];
    // the first histogram is cleared while the loads are in flight
    for (int i = tid; i < kSelKeyBins; i += kSelThreads) s_hist[i] = 0;
    if (tid == 0) s_res[3] = 0;
    __syncthreads();
    const int n = max(0, min(len_b, P));
    const int keff = min(k, n);
#pragma unroll
    for (int j = 0; j < PER; ++j)
        if (tid + j * kSelThreads >= n) v[j] = -1;     // valid scores are >= 0

    int T = 0x7FFFFFFF, needT = 0;
    bool all_ties = true;                     // every entry with s == T is taken
    if (keff > 0) {
        // pass 0: float-like key, fine enough that the atomics rarely collide;
        // masked entries count in bins past the key range (256 of them, one
        // per lane of a wave, so they do not collide either), never read
        const int spill = kSelKeyBins + (tid & 255);
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int key = sel_key(v[j]);          // defined for any int; used if v >= 0
            atomicAdd(&s_hist[v[j] >= 0 ? key : spill], 1u);
        }
        __syncthreads();
        sel_find_bin(s_hist, kSelKeyBins, keff, s_tmp, s_res);
        const int kb = s_res[0];
        int need = keff - s_res[1];
        int cnt = (int)s_hist[kb];            // entries inside the bin
        int lo, hi;
        if (kb < 128) {
            lo = hi = kb;
        } else {
            const int e = (kb >> 7) + 6;
            lo = (128 + (kb & 127)) << (e - 7);
            hi = lo + (1 << (e - 7)) - 1;
        }
        if (s_res[1] + cnt <= kSelThreads) {  // uniform: the usual case
            select_compacted(v, pos, lo, hi, cnt, need, keff, s_res[1] + cnt, k,
                             sel_pos + (size_t)b * k, sel_len + b, s_hist, s_tmp, s_res, s_cnt,
                             s_pre, s_cs, s_cp);
            return;
        }
        // 13-bit refinement passes until the bin is one value or holds <= kSelLast
        while (lo < hi && cnt > kSelLast) {
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
            cnt = (int)s_hist[d];
            const int nlo = lo + (d << sh);
            const int nhi = sub_range_hi(nlo, sh, hi);
            lo = nlo;
            hi = nhi;
        }
        if (lo < hi) {
            // <= kSelLast entries in [lo, hi]: gather their scores, one per
            // thread (one LDS atomic per wave for the slots), and take the last
            // digits on them
            __syncthreads();
            uint64_t min_[PER];
            int wcount = 0;
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                min_[j] = __ballot(v[j] >= lo && v[j] <= hi);
                wcount += __popcll(min_[j]);
            }
            int first = 0;
            if (lane == 0 && wcount) first = atomicAdd(&s_res[3], wcount);
            first = __builtin_amdgcn_readfirstlane(first);
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                const bool in = (min_[j] >> lane) & 1ull;
                const int slot = first + lane_rank64(min_[j]);
                if (in && slot < kSelLast) s_cs[slot] = v[j];
                first += __popcll(min_[j]);
            }
            __syncthreads();
            narrow_to_value(tid < cnt ? s_cs[tid] : -1, lo, hi, need, cnt, s_hist, s_res);
        }
        T = lo;
        needT = need;
        all_ties = need == cnt;
    }

    // ordered compaction over entries i = tid + 1024 j (slot j, then thread);
    // ties at T are ranked in list order only when some of them are dropped
    bool take[PER];
    if (all_ties) {
#pragma unroll
        for (int j = 0; j < PER; ++j) take[j] = v[j] >= 0 && v[j] >= T;
    } else {
        uint64_t meq[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            meq[j] = __ballot(v[j] >= 0 && v[j] == T);
            if (lane == 0) s_cnt[j * kSelWaves + wave] = __popcll(meq[j]);
        }
        slot_wave_scan(s_cnt, s_pre);
        int base[PER];
        wave_prefixes(s_pre, base);
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const bool eq = (meq[j] >> lane) & 1ull;
            const int eq_rank = base[j] + lane_rank64(meq[j]);
            take[j] = (v[j] > T) || (eq && eq_rank < needT);
        }
        __syncthreads();
    }
    uint64_t mt[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        mt[j] = __ballot(take[j]);
        if (lane == 0) s_cnt[j * kSelWaves + wave] = __popcll(mt[j]);
    }
    slot_wave_scan(s_cnt, s_pre);
    int obase[PER];
    wave_prefixes(s_pre, obase);
    int* out = sel_pos + (size_t)b * k;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        if (take[j]) {
            const int o = obase[j] + lane_rank64(mt[j]);
            if (o < keff) out[o] = pos[j];
        }
    }
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
