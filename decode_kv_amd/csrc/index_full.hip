// csa2_index_full: Full-mode index scan and candidate pool
// ("DeepSeek V4.1-Flash 552B runs like 16B (CED)", "Act 2": the first
// full-mode indexing layer searches the whole context and builds a candidate
// pool; "How DeepSeek V4.1 Flash Actually Works", item 2: up to 16,384
// candidate positions).
//
// Pipeline (all sequences of the batch at once, tiles of 2,048 positions):
//   1. prep      zero the histograms, per-sequence E, P_eff and tile ranges
//   2. score     stream the int8 keys once, int8 MFMA scoring, store int32
//                scores, LDS histogram of a 12-bit float-like key
//   3. resolve   per sequence: the histogram bin holding the P_eff-th score
//   4-7. refine  two more histogram passes over the scores in that bin
//                (11 bits each) until the threshold score T is exact
//   8. count     per tile: #(s > T) and #(s == T)
//   9. offsets   per sequence: exclusive prefix of the tile counts
//  10. write     ordered compaction: s > T, plus the first need_T ties in
//                position order; ascending positions, tail -1
// The result is exact and independent of the launch shape.
#include "abi_common.h"
#include "common.h"

namespace csa2 {

constexpr int kTile = 2048;
constexpr int kScanThreads = 256;
constexpr int kKeyBins = 3072;   // float-like key of a score < 2^30
constexpr int kRefBins = 2048;   // 11-bit refinement digit
constexpr int kMaxBatch = 4096;

struct FullState {
    int E;       // eligible positions
    int Peff;    // pool size
    int tile0;   // first global tile of this sequence
    int ntiles;  // tiles of this sequence
    int lo, hi;  // score interval known to hold the threshold
    int shift;   // bin shift of the next refinement pass
    int need;    // entries still to take from [lo, hi]
    int done;    // T / needT final
    int T;       // take s > T ...
    int needT;   // ... plus the first needT with s == T
    int pad[5];
};
static_assert(sizeof(FullState) == 64, "FullState size");

struct FullWs {
    FullState* st;
    uint32_t* hist1;   // [B][kKeyBins]
    uint32_t* hist2;   // [B][kRefBins]
    uint32_t* hist3;   // [B][kRefBins]
    int* tile_cnt;     // [Tmax][2]
    int* tile_off;     // [Tmax][2]
    int* meta;         // [0] = total tiles
    int* scores;       // [Tmax * kTile]
};

static long long full_tile_bound(int B, long long total_len) {
    return total_len / kTile + B + 1;
}

static FullWs carve_full_ws(void* ws, int B, long long total_len) {
    const long long T = full_tile_bound(B, total_len);
    char* p = reinterpret_cast<char*>(ws);
    FullWs w;
    size_t off = 0;
    w.st = reinterpret_cast<FullState*>(p + off);
    off = round_up(off + sizeof(FullState) * (size_t)B, 256);
    w.hist1 = reinterpret_cast<uint32_t*>(p + off);
    off = round_up(off + 4ull * B * kKeyBins, 256);
    w.hist2 = reinterpret_cast<uint32_t*>(p + off);
    off = round_up(off + 4ull * B * kRefBins, 256);
    w.hist3 = reinterpret_cast<uint32_t*>(p + off);
    off = round_up(off + 4ull * B * kRefBins, 256);
    w.tile_cnt = reinterpret_cast<int*>(p + off);
    off = round_up(off + 8ull * T, 256);
    w.tile_off = reinterpret_cast<int*>(p + off);
    off = round_up(off + 8ull * T, 256);
    w.meta = reinterpret_cast<int*>(p + off);
    off = round_up(off + 256, 256);
    w.scores = reinterpret_cast<int*>(p + off);
    return w;
}

size_t index_full_ws_bytes(int B, long long total_len, int P) {
    (void)P;
    const long long T = full_tile_bound(B, total_len);
    size_t off = 0;
    off = round_up(off + sizeof(FullState) * (size_t)B, 256);
    off = round_up(off + 4ull * B * kKeyBins, 256);
    off = round_up(off + 4ull * B * kRefBins, 256);
    off = round_up(off + 4ull * B * kRefBins, 256);
    off = round_up(off + 8ull * T, 256);
    off = round_up(off + 8ull * T, 256);
    off = round_up(off + 256, 256);
    off = round_up(off + 4ull * (size_t)T * kTile, 256);
    return off;
}

// Monotone 12-bit key of a score: exact below 128, otherwise the exponent and
// the 7 bits below the leading one.
__device__ __forceinline__ int score_key(int s) {
    if (s < 128) return s < 0 ? 0 : s;              // (negative only for invalid weights)
    const int e = 31 - __clz(s);                    // 7 .. 29 for valid inputs
    const int k = ((e - 6) << 7) | ((s >> (e - 7)) & 127);
    return k < kKeyBins ? k : kKeyBins - 1;
}

__device__ __forceinline__ void key_interval(int key, int& lo, int& hi) {
    if (key < 128) {
        lo = hi = key;
        return;
    }
    const int e = (key >> 7) + 6;
    const int m = key & 127;
    lo = (128 + m) << (e - 7);
    hi = lo + (1 << (e - 7)) - 1;
}

__device__ __forceinline__ int next_shift(int lo, int hi) {
    const unsigned width = (unsigned)(hi - lo) + 1u;   // >= 2 when called
    const int bits = 32 - __clz(width - 1u);            // ceil(log2 width)
    return bits > 11 ? bits - 11 : 0;
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

// ---- 1. prep ---------------------------------------------------------------
__global__ __launch_bounds__(kScanThreads) void full_prep_kernel(
    const int* __restrict__ len, int B, int window, int P, FullWs w) {
    const size_t nzero = (size_t)B * (kKeyBins + 2 * kRefBins);
    // hist1, hist2, hist3 are consecutive and 256-aligned blocks
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < (size_t)B * kKeyBins;
         i += (size_t)gridDim.x * blockDim.x)
        w.hist1[i] = 0;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < (size_t)B * kRefBins;
         i += (size_t)gridDim.x * blockDim.x) {
        w.hist2[i] = 0;
        w.hist3[i] = 0;
    }
    (void)nzero;
    if (blockIdx.x != 0) return;
    __shared__ int s_nt[kMaxBatch];
    for (int b = threadIdx.x; b < B; b += blockDim.x) {
        const int L = len[b];
        const int E = L > window ? L - window : 0;
        s_nt[b] = (E + kTile - 1) / kTile;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int acc = 0;
        for (int b = 0; b < B; ++b) {
            const int nt = s_nt[b];
            s_nt[b] = acc;
            acc += nt;
        }
        w.meta[0] = acc;
    }
    __syncthreads();
    for (int b = threadIdx.x; b < B; b += blockDim.x) {
        const int L = len[b];
        const int E = L > window ? L - window : 0;
        FullState s;
        s.E = E;
        s.Peff = E < P ? E : P;
        s.tile0 = s_nt[b];
        s.ntiles = (E + kTile - 1) / kTile;
        s.lo = 0;
        s.hi = 0x7FFFFFFF;
        s.shift = 0;
        s.need = s.Peff;
        s.done = s.Peff == 0 ? 1 : 0;
        s.T = 0x7FFFFFFF;
        s.needT = 0;
        for (int i = 0; i < 5; ++i) s.pad[i] = 0;
        w.st[b] = s;
    }
}

// ---- 2. score + first histogram ---------------------------------------------
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
    const int8_t* kbase = keys + ((size_t)row_off[b] + p_tile) * kDk;
    int* sc_out = w.scores + (size_t)t * kTile;
    const int nvalid = min(kTile, st.E - p_tile);
    __syncthreads();

    for (int it = 0; it < kTile / (4 * 64); ++it) {
        const int base = 64 * (wave + 4 * it);                  // 64 tokens per wave step
        if (base >= nvalid) break;
        i32x4 kop[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            int tok = base + 16 * u + (l & 15);
            tok = tok < nvalid ? tok : 0;
            kop[u] = *reinterpret_cast<const i32x4*>(kbase + (size_t)tok * kDk + (l >> 4) * 16);
        }
        int sc[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) sc[u] = score_group16<NB>(qa, wr, kop[u]);
        const int g = l >> 4;
        const int mine = g == 0 ? sc[0] : (g == 1 ? sc[1] : (g == 2 ? sc[2] : sc[3]));
        const int tok = base + l;
        if (tok < nvalid) {
            sc_out[tok] = mine;
            atomicAdd(&s_hist[score_key(mine)], 1u);
        }
    }
    __syncthreads();
    uint32_t* gh = w.hist1 + (size_t)b * kKeyBins;
    for (int i = threadIdx.x; i < kKeyBins; i += kScanThreads) {
        const uint32_t c = s_hist[i];
        if (c) atomicAdd(&gh[i], c);
    }
}

// ---- 3/5/7. resolve: find the bin holding the threshold -----------------------
// pass 1: bins are score_key values; passes 2 and 3: (s - lo) >> shift.
template <int NBINS, bool FIRST>
__global__ __launch_bounds__(kScanThreads) void full_resolve_kernel(const uint32_t* __restrict__ hist,
                                                                    FullWs w) {
    constexpr int PER = NBINS / kScanThreads;
    __shared__ uint32_t s_sum[kScanThreads];
    const int b = blockIdx.x;
    FullState st = w.st[b];
    if (st.done) return;
    const uint32_t* h = hist + (size_t)b * NBINS;
    uint32_t c[PER];
    uint32_t mysum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        c[i] = h[threadIdx.x * PER + i];
        mysum += c[i];
    }
    s_sum[threadIdx.x] = mysum;
    __syncthreads();
    // suffix sum over threads above this one (bins above this thread's range)
    uint32_t above = 0;
    for (int j = threadIdx.x + 1; j < kScanThreads; ++j) above += s_sum[j];
    const uint32_t need = (uint32_t)st.need;
    if (above < need && need <= above + mysum) {
        uint32_t acc = above;
        for (int i = PER - 1; i >= 0; --i) {
            if (acc + c[i] >= need) {
                const int bin = threadIdx.x * PER + i;
                int lo, hi;
                if (FIRST) {
                    key_interval(bin, lo, hi);
                } else {
                    lo = st.lo + (bin << st.shift);
                    hi = lo + (1 << st.shift) - 1;
                    if (hi > st.hi || hi < lo) hi = st.hi;
                }
                st.need = (int)(need - acc);
                st.lo = lo;
                st.hi = hi;
                if ((uint32_t)st.need == c[i]) {        // the whole bin is taken
                    st.done = 1;
                    st.T = lo - 1;
                    st.needT = 0;
                } else if (lo == hi) {                  // exact threshold
                    st.done = 1;
                    st.T = lo;
                    st.needT = st.need;
                } else {
                    st.shift = next_shift(lo, hi);
                }
                w.st[b] = st;
                break;
            }
            acc += c[i];
        }
    }
}

// ---- 4/6. refine: histogram of the scores inside [lo, hi] ---------------------
__global__ __launch_bounds__(kScanThreads) void full_refine_kernel(uint32_t* __restrict__ hist,
                                                                   int B, FullWs w) {
    __shared__ uint32_t s_hist[kRefBins];
    __shared__ int s_b;
    const int t = blockIdx.x;
    if (t >= w.meta[0]) return;
    const int b = find_tile_seq(w.st, B, t, &s_b);
    if (b < 0) return;
    const FullState st = w.st[b];
    if (st.done) return;
    for (int i = threadIdx.x; i < kRefBins; i += kScanThreads) s_hist[i] = 0;
    __syncthreads();
    const int p_tile = (t - st.tile0) * kTile;
    const int nvalid = min(kTile, st.E - p_tile);
    const int* sc = w.scores + (size_t)t * kTile;
    for (int i = threadIdx.x; i < nvalid; i += kScanThreads) {
        const int s = sc[i];
        if (s >= st.lo && s <= st.hi)
            atomicAdd(&s_hist[min((s - st.lo) >> st.shift, kRefBins - 1)], 1u);
    }
    __syncthreads();
    uint32_t* gh = hist + (size_t)b * kRefBins;
    for (int i = threadIdx.x; i < kRefBins; i += kScanThreads) {
        const uint32_t c = s_hist[i];
        if (c) atomicAdd(&gh[i], c);
    }
}

// ---- 8. count ------------------------------------------------------------------
__global__ __launch_bounds__(kScanThreads) void full_count_kernel(int B, FullWs w) {
    __shared__ int s_b;
    __shared__ int s_red[2][kScanThreads / kWave];
    const int t = blockIdx.x;
    if (t >= w.meta[0]) return;
    const int b = find_tile_seq(w.st, B, t, &s_b);
    if (b < 0) return;
    const FullState st = w.st[b];
    const int p_tile = (t - st.tile0) * kTile;
    const int nvalid = min(kTile, st.E - p_tile);
    const int* sc = w.scores + (size_t)t * kTile;
    int gt = 0, eq = 0;
    for (int i = threadIdx.x; i < nvalid; i += kScanThreads) {
        const int s = sc[i];
        gt += s > st.T;
        eq += s == st.T;
    }
    for (int o = 32; o > 0; o >>= 1) {
        gt += __shfl_xor(gt, o);
        eq += __shfl_xor(eq, o);
    }
    if (lane_id() == 0) {
        s_red[0][threadIdx.x / kWave] = gt;
        s_red[1][threadIdx.x / kWave] = eq;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int g = 0, e = 0;
        for (int i = 0; i < kScanThreads / kWave; ++i) {
            g += s_red[0][i];
            e += s_red[1][i];
        }
        w.tile_cnt[2 * t] = g;
        w.tile_cnt[2 * t + 1] = e;
    }
}

// ---- 9. offsets: exclusive prefix over each sequence's tiles ---------------------
__global__ __launch_bounds__(kScanThreads) void full_offsets_kernel(FullWs w) {
    __shared__ int s_g[kScanThreads], s_e[kScanThreads];
    const int b = blockIdx.x;
    const FullState st = w.st[b];
    int carry_g = 0, carry_e = 0;
    for (int base = 0; base < st.ntiles; base += kScanThreads) {
        const int i = base + threadIdx.x;
        const int t = st.tile0 + i;
        const int g = i < st.ntiles ? w.tile_cnt[2 * t] : 0;
        const int e = i < st.ntiles ? w.tile_cnt[2 * t + 1] : 0;
        s_g[threadIdx.x] = g;
        s_e[threadIdx.x] = e;
        __syncthreads();
        for (int o = 1; o < kScanThreads; o <<= 1) {   // inclusive Hillis-Steele scan
            const int ag = threadIdx.x >= o ? s_g[threadIdx.x - o] : 0;
            const int ae = threadIdx.x >= o ? s_e[threadIdx.x - o] : 0;
            __syncthreads();
            s_g[threadIdx.x] += ag;
            s_e[threadIdx.x] += ae;
            __syncthreads();
        }
        if (i < st.ntiles) {
            w.tile_off[2 * t] = carry_g + s_g[threadIdx.x] - g;
            w.tile_off[2 * t + 1] = carry_e + s_e[threadIdx.x] - e;
        }
        carry_g += s_g[kScanThreads - 1];
        carry_e += s_e[kScanThreads - 1];
        __syncthreads();
    }
}

// Exclusive block-wide prefix sum of one int per thread (256 threads).
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
    for (int i = 0; i < kScanThreads / kWave; ++i) {
        const int c = s_tmp[i];
        if (i < wv) before += c;
        total += c;
    }
    __syncthreads();
    return before + x - v;
}

// ---- 10. write: ordered compaction of the pool ------------------------------------
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
    const int eq_before = block_exclusive_scan(n_eq, s_tmp, tot) + w.tile_off[2 * t + 1];
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
    const int tile_eq = w.tile_off[2 * t + 1];
    int base = w.tile_off[2 * t] + (tile_eq < st.needT ? tile_eq : st.needT);
    base += block_exclusive_scan(n_sel, s_tmp, tot);
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
    if (max_len >= (1ll << 31)) return fail(CSA2_ERR_UNSUPPORTED, "csa2_index_full: max_len >= 2^31");
    if (!aligned(q, 16) || !aligned(keys, 16) || !aligned(row_off, 8) || !aligned(len, 4))
        return fail(CSA2_ERR_INVALID, "csa2_index_full: misaligned pointer");
    const size_t need = index_full_ws_bytes(B, total_len, P);
    if (!ws || ws_bytes < need || !aligned(ws, 256))
        return fail(CSA2_ERR_WORKSPACE, "csa2_index_full: workspace needs %zu bytes (256-aligned)",
                    need);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    FullWs fw = carve_full_ws(ws, B, total_len);
    const unsigned tiles = (unsigned)full_tile_bound(B, total_len);
    const dim3 blk(kScanThreads);

    const unsigned prep_grid = (unsigned)std::min<long long>(1024, ((long long)B * kKeyBins + 1023) / 1024);
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

    hipLaunchKernelGGL((full_resolve_kernel<kKeyBins, true>), dim3(B), blk, 0, s, fw.hist1, fw);
    hipLaunchKernelGGL(full_refine_kernel, dim3(tiles), blk, 0, s, fw.hist2, B, fw);
    hipLaunchKernelGGL((full_resolve_kernel<kRefBins, false>), dim3(B), blk, 0, s, fw.hist2, fw);
    hipLaunchKernelGGL(full_refine_kernel, dim3(tiles), blk, 0, s, fw.hist3, B, fw);
    hipLaunchKernelGGL((full_resolve_kernel<kRefBins, false>), dim3(B), blk, 0, s, fw.hist3, fw);
    hipLaunchKernelGGL(full_count_kernel, dim3(tiles), blk, 0, s, B, fw);
    hipLaunchKernelGGL(full_offsets_kernel, dim3(B), blk, 0, s, fw);
    const unsigned wgrid = tiles > (unsigned)B ? tiles : (unsigned)B;
    hipLaunchKernelGGL(full_write_kernel, dim3(wgrid), blk, 0, s, B, P, pool_pos, pool_score,
                       pool_len, fw);
    return launch_status("csa2_index_full launch");
}
