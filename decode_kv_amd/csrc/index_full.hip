// csa2_index_full: Full-mode index scan and candidate pool
// ("DeepSeek V4.1-Flash 552B runs like 16B (CED)", "Act 2": the first
// full-mode indexing layer searches the whole context and builds a candidate
// pool; "How DeepSeek V4.1 Flash Actually Works", item 2: up to 16,384
// candidate positions).
//
// Five kernels, all sequences of the batch at once, tiles of 1,024 positions:
//   1. prep       zero the first-level histogram and candidate counters;
//                 per-sequence E, P_eff and tile range
//   2. score      stream the int8 keys once (each wave issues all of its tile
//                 loads at once, 16 KB in flight), int8 MFMA scoring, int32 scores to
//                 scratch, LDS histogram of a float-like key (exponent + 5
//                 mantissa bits, 832 bins), flushed with one atomic per
//                 non-empty bin
//   3. gather     every tile finds the bin holding the P_eff-th score from the
//                 histogram, counts its entries above that bin and appends the
//                 entries inside it to a candidate list (one atomic per tile)
//   4. threshold  one workgroup per sequence: exact radix select over the
//                 candidates (13-bit digits) gives the threshold T and the
//                 number of ties at T to keep; per-tile counts and an
//                 exclusive prefix give every tile its output offsets
//   5. write      ordered compaction: s > T, plus the first ties in position
//                 order; ascending positions, tail -1
// The result is exact and independent of the launch shape.
#include "abi_common.h"
#include "common.h"

namespace csa2 {

constexpr int kTile = 1024;
constexpr int kScanThreads = 256;
constexpr int kKeyBins = 832;            // float-like key of a score < 2^31
constexpr int kThrThreads = 1024;
constexpr int kThrWaves = kThrThreads / kWave;
constexpr int kMaxTilesPerSeq = 8192;    // LDS tile counters of the threshold kernel (8M positions)
constexpr int kRefBins = 8192;           // 13-bit refinement digit
constexpr int kMaxBatch = 4096;

struct FullState {
    int E;       // eligible positions
    int Peff;    // pool size
    int tile0;   // first global tile of this sequence
    int ntiles;  // tiles of this sequence
    int cand0;   // first slot of this sequence's candidate list
    int T;       // take s > T ...
    int needT;   // ... plus the first needT entries with s == T
    int pad;
};
static_assert(sizeof(FullState) == 32, "FullState size");

struct FullWs {
    FullState* st;        // [B]
    uint32_t* hist;       // [B][kKeyBins]
    int* cand_cnt;        // [B]
    int* tile_above;      // [Tmax] entries of the tile above the threshold bin
    int* tile_off;        // [Tmax][2] output offsets among s > T and among s == T
    int* meta;            // [0] total tiles
    int2* cand;           // [total_len] (score, position)
    int* scores;          // [Tmax * kTile]
};

static long long full_tile_bound(int B, long long total_len) {
    return total_len / kTile + B + 1;
}

static size_t full_ws_layout(int B, long long total_len, char* base, FullWs* w) {
    const long long T = full_tile_bound(B, total_len);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = round_up(off + bytes, 256);
        return base ? base + at : nullptr;
    };
    FullWs x;
    x.st = reinterpret_cast<FullState*>(take(sizeof(FullState) * (size_t)B));
    x.hist = reinterpret_cast<uint32_t*>(take(4ull * B * kKeyBins));
    x.cand_cnt = reinterpret_cast<int*>(take(4ull * B));
    x.tile_above = reinterpret_cast<int*>(take(4ull * T));
    x.tile_off = reinterpret_cast<int*>(take(8ull * T));
    x.meta = reinterpret_cast<int*>(take(256));
    x.cand = reinterpret_cast<int2*>(take(8ull * (size_t)(total_len > 0 ? total_len : 1)));
    x.scores = reinterpret_cast<int*>(take(4ull * (size_t)T * kTile));
    if (w) *w = x;
    return off;
}

size_t index_full_ws_bytes(int B, long long total_len, int P) {
    (void)P;
    return full_ws_layout(B, total_len, nullptr, nullptr);
}

// Monotone key of a score: exact below 32, otherwise the exponent and the 5
// bits below the leading one (relative bin width 1/32).  Scores of valid
// inputs are < 2^30, so the key stays below 26 * 32 = 832.
__device__ __forceinline__ int score_key(int s) {
    if (s < 32) return s < 0 ? 0 : s;                  // negative only for invalid weights
    const int e = 31 - __clz(s);
    const int k = ((e - 4) << 5) | ((s >> (e - 5)) & 31);
    return k < kKeyBins ? k : kKeyBins - 1;
}

__device__ __forceinline__ void key_interval(int key, int& lo, int& hi) {
    if (key < 32) {
        lo = hi = key;
        return;
    }
    const int e = (key >> 5) + 4;
    lo = (32 + (key & 31)) << (e - 5);
    hi = (key == kKeyBins - 1) ? 0x7FFFFFFF : lo + (1 << (e - 5)) - 1;
}

// Sequence owning global tile t (threads of the block cooperate; result in LDS).
__device__ int find_tile_seq(const FullState* __restrict__ st, int B, int t, int* s_b) {
    if (threadIdx.x == 0) *s_b = -1;
    __syncthreads();
    for (int b = threadIdx.x; b < B; b += blockDim.x) {
        const int t0 = st[b].tile0;
        if (t >= t0 && t < t0 + st[b].ntiles) *s_b = b;
    }
    __syncthreads();
    return *s_b;
}

// Exclusive prefix sum of one int per thread over the block.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_tmp, int& total) {
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
    for (int i = 0; i < NT / kWave; ++i) {
        const int c = s_tmp[i];
        if (i < wv) before += c;
        total += c;
    }
    __syncthreads();
    return before + x - v;
}

// Bin holding the need-th largest entry of a histogram (bins ascending in
// value); every thread gets (bin, entries in higher bins).  Requires
// 1 <= need <= total count.
template <int NT, int PER>
__device__ __forceinline__ void find_bin(const uint32_t* h, int nb, int need, int* s_tmp,
                                         int* s_res, int& bin_out, int& above_out) {
    const int r = NT - 1 - threadIdx.x;          // thread 0 owns the highest bins
    uint32_t c[PER];
    int mysum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int bin = r * PER + i;
        c[i] = bin < nb ? h[bin] : 0u;
        mysum += (int)c[i];
    }
    int tot;
    const int above = block_exclusive_scan<NT>(mysum, s_tmp, tot);
    if (above < need && need <= above + mysum) {
        int acc = above;
#pragma unroll
        for (int i = PER - 1; i >= 0; --i) {
            if (acc < need && need <= acc + (int)c[i]) {
                s_res[0] = r * PER + i;
                s_res[1] = acc;
            }
            acc += (int)c[i];
        }
    }
    __syncthreads();
    bin_out = s_res[0];
    above_out = s_res[1];
    __syncthreads();
}

// ---- 1. prep ---------------------------------------------------------------
__global__ __launch_bounds__(kScanThreads) void full_prep_kernel(
    const int* __restrict__ len, int B, int window, int P, FullWs w) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < (size_t)B * kKeyBins;
         i += (size_t)gridDim.x * blockDim.x)
        w.hist[i] = 0;
    if (blockIdx.x != 0) return;
    __shared__ int s_tmp[kScanThreads / kWave];
    __shared__ int s_carry[2];
    if (threadIdx.x == 0) s_carry[0] = s_carry[1] = 0;
    __syncthreads();
    for (int base = 0; base < B; base += kScanThreads) {   // uniform trip count
        const int b = base + threadIdx.x;
        int E = 0;
        if (b < B) {
            const int L = len[b];
            E = L > window ? L - window : 0;
        }
        const int nt = (E + kTile - 1) / kTile;
        int tot_t, tot_e;
        const int pre_t = block_exclusive_scan<kScanThreads>(nt, s_tmp, tot_t);
        const int pre_e = block_exclusive_scan<kScanThreads>(E, s_tmp, tot_e);
        if (b < B) {
            FullState s;
            s.E = E;
            s.Peff = E < P ? E : P;
            s.tile0 = s_carry[0] + pre_t;
            s.ntiles = nt;
            s.cand0 = s_carry[1] + pre_e;
            s.T = 0x7FFFFFFF;
            s.needT = 0;
            s.pad = 0;
            w.st[b] = s;
            w.cand_cnt[b] = 0;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            s_carry[0] += tot_t;
            s_carry[1] += tot_e;
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) w.meta[0] = s_carry[0];
}

// ---- 2. score + first-level histogram ----------------------------------------
template <int NB>
__global__ __launch_bounds__(kScanThreads) void full_score_kernel(
    const int8_t* __restrict__ q, const int8_t* __restrict__ wts,
    const int8_t* __restrict__ keys, const long long* __restrict__ row_off, int B, int H,
    FullWs w) {
    __shared__ uint32_t s_hist[kKeyBins];
    __shared__ int s_b;
    const int t = blockIdx.x;
    if (t >= w.meta[0]) return;
    const int b = find_tile_seq(w.st, B, t, &s_b);
    if (b < 0) return;
    const FullState st = w.st[b];
    for (int i = threadIdx.x; i < kKeyBins; i += kScanThreads) s_hist[i] = 0;

    i32x4 qa[NB];
    uint32_t wr[NB][4];
    load_index_query<NB>(q + (size_t)b * H * kDk, wts + (size_t)b * H, H, qa, wr);

    const int l = lane_id();
    const int wave = threadIdx.x / kWave;
    const int p_tile = (t - st.tile0) * kTile;                 // first position
    const int8_t* kbase = keys + ((size_t)row_off[b] + p_tile) * kDk + (l >> 4) * 16;
    int* sc_out = w.scores + (size_t)t * kTile;
    const int nvalid = min(kTile, st.E - p_tile);
    // wave w scores tokens [256w, 256w + 256): 16 groups of 16, all loads issued
    // before the first MFMA so 16 KB per wave are in flight
    constexpr int kGroups = kTile / (4 * 16);
    const int t0 = (kTile / 4) * wave;
    i32x4 kop[kGroups];
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kGroups; ++u) {
        int tok = t0 + 16 * u + (l & 15);
        tok = tok < nvalid ? tok : 0;
        kop[u] = *reinterpret_cast<const i32x4*>(kbase + (size_t)tok * kDk);
    }
#pragma unroll
    for (int it = 0; it < kGroups / 4; ++it) {
        if (t0 + 64 * it >= nvalid) break;                     // wave-uniform
        int sc[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) sc[u] = score_group16<NB>(qa, wr, kop[4 * it + u]);
        const int g = l >> 4;
        const int mine = g == 0 ? sc[0] : (g == 1 ? sc[1] : (g == 2 ? sc[2] : sc[3]));
        const int tok = t0 + 64 * it + l;
        if (tok < nvalid) {
            sc_out[tok] = mine;
            atomicAdd(&s_hist[score_key(mine)], 1u);
        }
    }
    __syncthreads();
    uint32_t* gh = w.hist + (size_t)b * kKeyBins;
    for (int i = threadIdx.x; i < kKeyBins; i += kScanThreads) {
        const uint32_t c = s_hist[i];
        if (c) atomicAdd(&gh[i], c);
    }
}

// ---- 3. gather: entries above / inside the threshold bin ------------------------
__global__ __launch_bounds__(kScanThreads) void full_gather_kernel(int B, FullWs w) {
    __shared__ int s_b;
    __shared__ int s_tmp[kScanThreads / kWave];
    __shared__ int s_res[2];
    const int t = blockIdx.x;
    if (t >= w.meta[0]) return;
    const int b = find_tile_seq(w.st, B, t, &s_b);
    if (b < 0) return;
    const FullState st = w.st[b];
    int kb, above;
    find_bin<kScanThreads, (kKeyBins + kScanThreads - 1) / kScanThreads>(
        w.hist + (size_t)b * kKeyBins, kKeyBins, st.Peff, s_tmp, s_res, kb, above);
    int lo, hi;
    key_interval(kb, lo, hi);
    const int p_tile = (t - st.tile0) * kTile;
    const int nvalid = min(kTile, st.E - p_tile);
    const int* sc = w.scores + (size_t)t * kTile;
    constexpr int PER = kTile / kScanThreads;
    int v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int i = threadIdx.x + j * kScanThreads;
        v[j] = i < nvalid ? sc[i] : -1;
    }
    // per-thread counts of entries above / inside the bin, packed in one scan
    int n_above = 0, n_in = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        n_above += v[j] > hi;
        n_in += v[j] >= lo && v[j] <= hi;
    }
    int tot;
    const int pre = block_exclusive_scan<kScanThreads>((n_in << 16) | n_above, s_tmp, tot);
    const int tot_in = tot >> 16;
    if (threadIdx.x == 0) {
        w.tile_above[t] = tot & 0xFFFF;
        s_res[0] = tot_in ? atomicAdd(&w.cand_cnt[b], tot_in) : 0;   // one atomic per tile
    }
    __syncthreads();
    int slot = s_res[0] + (pre >> 16);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        if (v[j] >= lo && v[j] <= hi) {
            if (slot < st.E)                           // at most E candidates
                w.cand[(size_t)st.cand0 + slot] =
                    make_int2(v[j], p_tile + (int)threadIdx.x + j * kScanThreads);
            ++slot;
        }
    }
}

// ---- 4. threshold: exact select among the candidates, tile offsets ---------------
__global__ __launch_bounds__(kThrThreads) void full_threshold_kernel(FullWs w) {
    __shared__ uint32_t s_hist[kRefBins];
    __shared__ uint32_t s_cgt[kMaxTilesPerSeq];
    __shared__ uint32_t s_ceq[kMaxTilesPerSeq];
    __shared__ int s_tmp[kThrWaves];
    __shared__ int s_res[2];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const FullState st = w.st[b];
    if (st.Peff == 0) return;
    int kb, above;
    find_bin<kThrThreads, 1>(w.hist + (size_t)b * kKeyBins, kKeyBins, st.Peff, s_tmp, s_res, kb,
                             above);
    int lo, hi;
    key_interval(kb, lo, hi);
    int need = st.Peff - above;
    const int nc = min(w.cand_cnt[b], st.E);
    const int2* cand = w.cand + st.cand0;
    constexpr int PER = 16;
    constexpr int CHUNK = kThrThreads * PER;
    // this thread's tiles' above-bin counts, loaded early
    constexpr int TPT = kMaxTilesPerSeq / kThrThreads;
    int above_t[TPT];
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
        const int i = tid * TPT + u;
        above_t[u] = i < st.ntiles ? w.tile_above[st.tile0 + i] : 0;
    }
    // first chunk of candidates stays in registers for every pass
    int2 c0v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int i = tid + j * kThrThreads;
        c0v[j] = i < nc ? cand[i] : make_int2(-1, 0);
    }
    // refine [lo, hi] with 13-bit digits until one value remains
    while (lo < hi) {                                  // uniform: lo, hi from LDS
        const unsigned width = (unsigned)(hi - lo) + 1u;
        const int bits = 32 - __clz(width - 1u);
        const int sh = bits > 13 ? bits - 13 : 0;
        const int nb = (int)(((width - 1u) >> sh) + 1u);
        for (int i = tid; i < nb; i += kThrThreads) s_hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < PER; ++j)
            if (c0v[j].x >= lo && c0v[j].x <= hi) atomicAdd(&s_hist[(c0v[j].x - lo) >> sh], 1u);
        for (int c0 = CHUNK; c0 < nc; c0 += CHUNK) {   // many candidates: stream the rest
            int v[PER];
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                const int i = c0 + tid + j * kThrThreads;
                v[j] = i < nc ? cand[i].x : -1;
            }
#pragma unroll
            for (int j = 0; j < PER; ++j)
                if (v[j] >= lo && v[j] <= hi) atomicAdd(&s_hist[(v[j] - lo) >> sh], 1u);
        }
        __syncthreads();
        int d, a;
        find_bin<kThrThreads, kRefBins / kThrThreads>(s_hist, nb, need, s_tmp, s_res, d, a);
        need -= a;
        const int nlo = lo + (d << sh);
        const int nhi = (sh == 0) ? nlo : min(hi, nlo + (1 << sh) - 1);
        lo = nlo;
        hi = nhi;
    }
    const int T = lo, needT = need;

    // per-tile counts of candidates above / at the threshold
    for (int i = tid; i < st.ntiles; i += kThrThreads) {
        s_cgt[i] = 0;
        s_ceq[i] = 0;
    }
    __syncthreads();
    auto count_tiles = [&](const int2 (&v)[PER]) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int tile = min(max(v[j].y, 0) / kTile, kMaxTilesPerSeq - 1);
            if (v[j].x > T) atomicAdd(&s_cgt[tile], 1u);
            else if (v[j].x >= 0 && v[j].x == T) atomicAdd(&s_ceq[tile], 1u);
        }
    };
    count_tiles(c0v);
    for (int c0 = CHUNK; c0 < nc; c0 += CHUNK) {
        int2 v[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int i = c0 + tid + j * kThrThreads;
            v[j] = i < nc ? cand[i] : make_int2(-1, 0);
        }
        count_tiles(v);
    }
    __syncthreads();
    // exclusive prefix over this sequence's tiles, TPT tiles per thread
    int gl[TPT], el[TPT];
    int gs = 0, es = 0;
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
        const int i = tid * TPT + u;
        gl[u] = i < st.ntiles ? above_t[u] + (int)s_cgt[i] : 0;
        el[u] = i < st.ntiles ? (int)s_ceq[i] : 0;
        gs += gl[u];
        es += el[u];
    }
    int tot;
    int og = block_exclusive_scan<kThrThreads>(gs, s_tmp, tot);
    int oe = block_exclusive_scan<kThrThreads>(es, s_tmp, tot);
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
        const int i = tid * TPT + u;
        if (i < st.ntiles) {
            w.tile_off[2 * (st.tile0 + i)] = og;
            w.tile_off[2 * (st.tile0 + i) + 1] = oe;
        }
        og += gl[u];
        oe += el[u];
    }
    if (tid == 0) {
        w.st[b].T = T;
        w.st[b].needT = needT;
    }
}

// ---- 5. write: ordered compaction of the pool ------------------------------------
__global__ __launch_bounds__(kScanThreads) void full_write_kernel(int B, int P,
                                                                  int* __restrict__ pool_pos,
                                                                  int* __restrict__ pool_score,
                                                                  int* __restrict__ pool_len,
                                                                  FullWs w) {
    __shared__ int s_b;
    __shared__ int s_tmp[kScanThreads / kWave];
    const int t = blockIdx.x;
    // tail fill of sequence t (each block handles at most one sequence's tail)
    if (t < B) {
        const int Peff = w.st[t].Peff;
        for (int i = Peff + threadIdx.x; i < P; i += kScanThreads) {
            pool_pos[(size_t)t * P + i] = -1;
            pool_score[(size_t)t * P + i] = -1;
        }
        if (threadIdx.x == 0) pool_len[t] = Peff;
    }
    if (t >= w.meta[0]) return;
    const int b = find_tile_seq(w.st, B, t, &s_b);
    if (b < 0) return;
    const FullState st = w.st[b];
    const int p_tile = (t - st.tile0) * kTile;
    const int nvalid = min(kTile, st.E - p_tile);
    const int* sc = w.scores + (size_t)t * kTile;
    constexpr int PER = kTile / kScanThreads;   // 8 contiguous positions per thread
    const int i0 = threadIdx.x * PER;
    int v[PER];
    int n_eq = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        v[j] = (i0 + j < nvalid) ? sc[i0 + j] : -1;   // scores are >= 0
        n_eq += (v[j] >= 0) & (v[j] == st.T);
    }
    int tot;
    const int tile_gt = w.tile_off[2 * t], tile_eq = w.tile_off[2 * t + 1];
    const int eq_before = block_exclusive_scan<kScanThreads>(n_eq, s_tmp, tot) + tile_eq;
    int n_sel = 0, eq_rank = eq_before;
    bool take[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        bool tk = false;
        if (v[j] < 0) tk = false;
        else if (v[j] > st.T) tk = true;
        else if (v[j] == st.T) {
            tk = eq_rank < st.needT;
            ++eq_rank;
        }
        take[j] = tk;
        n_sel += tk;
    }
    int base = tile_gt + (tile_eq < st.needT ? tile_eq : st.needT);
    base += block_exclusive_scan<kScanThreads>(n_sel, s_tmp, tot);
    int* out_p = pool_pos + (size_t)b * P;
    int* out_s = pool_score + (size_t)b * P;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        if (take[j]) {
            if (base < st.Peff) {            // always true for consistent inputs
                out_p[base] = p_tile + i0 + j;
                out_s[base] = v[j];
            }
            ++base;
        }
    }
}

}  // namespace csa2

using namespace csa2;

extern "C" int csa2_index_full(const signed char* q, const signed char* w,
                               const signed char* keys, const long long* row_off,
                               const int* len, int B, long long max_len, long long total_len,
                               int H, int Dk, int window, int P, int* pool_pos,
                               int* pool_score, int* pool_len, void* ws, size_t ws_bytes,
                               void* stream) {
    if (B < 0 || max_len < 0 || total_len < 0)
        return fail(CSA2_ERR_INVALID, "csa2_index_full: negative size");
    if (B > kMaxBatch) return fail(CSA2_ERR_UNSUPPORTED, "csa2_index_full: B > %d", kMaxBatch);
    if (B == 0) return CSA2_OK;
    if (!q || !w || !keys || !row_off || !len || !pool_pos || !pool_score || !pool_len)
        return fail(CSA2_ERR_INVALID, "csa2_index_full: null pointer");
    if (Dk != kDk) return fail(CSA2_ERR_UNSUPPORTED, "csa2_index_full: Dk must be 64");
    if (H < 1 || H > 64) return fail(CSA2_ERR_INVALID, "csa2_index_full: H must be in [1, 64]");
    if (P < 1 || window < 0) return fail(CSA2_ERR_INVALID, "csa2_index_full: P < 1 or window < 0");
    if (max_len > (long long)kMaxTilesPerSeq * kTile)
        return fail(CSA2_ERR_UNSUPPORTED, "csa2_index_full: max_len > %lld",
                    (long long)kMaxTilesPerSeq * kTile);
    if (!aligned(q, 16) || !aligned(keys, 16) || !aligned(row_off, 8) || !aligned(len, 4))
        return fail(CSA2_ERR_INVALID, "csa2_index_full: misaligned pointer");
    const size_t need = index_full_ws_bytes(B, total_len, P);
    if (!ws || ws_bytes < need || !aligned(ws, 256))
        return fail(CSA2_ERR_WORKSPACE, "csa2_index_full: workspace needs %zu bytes (256-aligned)",
                    need);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    FullWs fw;
    full_ws_layout(B, total_len, reinterpret_cast<char*>(ws), &fw);
    const unsigned tiles = (unsigned)full_tile_bound(B, total_len);
    const dim3 blk(kScanThreads);

    const unsigned prep_grid =
        (unsigned)std::min<long long>(64, ((long long)B * kKeyBins + 4095) / 4096);
    hipLaunchKernelGGL(full_prep_kernel, dim3(prep_grid), blk, 0, s, len, B, window, P, fw);
    if (int e = launch_status("full_prep")) return e;

    if (g_scan_ev_start) hipEventRecord(g_scan_ev_start, s);
    const int NB = (H + 15) / 16;
    const int8_t* q8 = reinterpret_cast<const int8_t*>(q);
    const int8_t* w8 = reinterpret_cast<const int8_t*>(w);
    const int8_t* k8 = reinterpret_cast<const int8_t*>(keys);
    switch (NB) {
        case 1: hipLaunchKernelGGL(full_score_kernel<1>, dim3(tiles), blk, 0, s, q8, w8, k8, row_off, B, H, fw); break;
        case 2: hipLaunchKernelGGL(full_score_kernel<2>, dim3(tiles), blk, 0, s, q8, w8, k8, row_off, B, H, fw); break;
        case 3: hipLaunchKernelGGL(full_score_kernel<3>, dim3(tiles), blk, 0, s, q8, w8, k8, row_off, B, H, fw); break;
        default: hipLaunchKernelGGL(full_score_kernel<4>, dim3(tiles), blk, 0, s, q8, w8, k8, row_off, B, H, fw); break;
    }
    if (int e = launch_status("full_score")) return e;
    if (g_scan_ev_stop) hipEventRecord(g_scan_ev_stop, s);

    hipLaunchKernelGGL(full_gather_kernel, dim3(tiles), blk, 0, s, B, fw);
    hipLaunchKernelGGL(full_threshold_kernel, dim3(B), dim3(kThrThreads), 0, s, fw);
    const unsigned wgrid = tiles > (unsigned)B ? tiles : (unsigned)B;
    hipLaunchKernelGGL(full_write_kernel, dim3(wgrid), blk, 0, s, B, P, pool_pos, pool_score,
                       pool_len, fw);
    return launch_status("csa2_index_full launch");
}
