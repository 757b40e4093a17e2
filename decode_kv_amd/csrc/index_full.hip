// csa2_index_full: Full-mode index scan and candidate pool.
// ("DeepSeek V4.1-Flash 552B runs like 16B (CED)", "Act 2": one pass over
// every cached position ranks the context once and yields the pool that the
// later indexing layers work from; "How DeepSeek V4.1 Flash Actually Works",
// item 2: that pool holds at most 16,384 positions.)  csa2_index_score
// exposes the scoring stage alone.
//
// Five kernels, all sequences of the batch at once, tiles of 1,024 positions
// (per-tile grids padded to a multiple of 8 tiles, so tile t of every grid
// row runs on the XCD whose L2 holds its scores), no returning device-wide
// atomics:
//   1. score      stream the int8 keys once (each wave issues all of its tile
//                 loads before scoring), int8 MFMA scoring, int32 scores to
//                 scratch, and a per-tile histogram of a float-like key
//                 (exponent + 5 mantissa bits, 832 bins) written with plain
//                 stores; workgroup 0 also writes the per-sequence layout
//   2. reduce     sum the per-tile histograms of each sequence (workgroups
//                 split the bins), clear the second-level histogram
//   3. gather     every tile finds the bin B1 holding the P_eff-th score,
//                 counts its entries above B1, copies the scores of its
//                 entries inside B1 to its own candidate slots (the first 16
//                 slot-major across tiles) and adds them to a 4,096-bin
//                 histogram of the next 12 bits inside B1 (atomics whose
//                 result is not waited for)
//   4. threshold  one workgroup per sequence, one tile per thread: B1's
//                 candidates are compacted into one LDS list (score, tile);
//                 the second-level histogram narrows B1 to one sub-bin; its
//                 scores (<= 1,024, else more 12-bit passes over the list)
//                 are gathered one per thread and 8-bit digit passes narrow
//                 them to the threshold T and the number of ties at T to
//                 keep (taken in position order); per-tile counts and an
//                 exclusive prefix give every tile its offsets
//   5. write      ordered compaction: s > T, plus the first ties in position
//                 order; ascending positions, tail -1
// With k > 0 the Full layer's own top-k selection comes out of the same
// chain: it is the first min(k, E) positions under the same order (the top k
// of the pool), so gather, threshold and write run a second target with
// P_eff = min(k, E) side by side with the pool (grid dimension y, separate
// candidate arrays) and no separate selection pass reads the pool back.
// The result is exact and independent of the launch shape.
//
// Verify blocks (csa2_index_full_block, csa2_index_score_block): kernel 1b
// scores all T tokens of a block from one load of the keys, and kernels 2-5
// run unchanged over the block's lists, T per sequence (one per token, each
// over its own eligible positions) or one (the best score over the block).
#include "abi_common.h"
#include "common.h"

namespace csa2 {

constexpr int kTile = 1024;
constexpr int kScanThreads = 256;
constexpr int kScoreThreads = 512;       // scoring kernel: 8 waves x 128 tokens
constexpr int kKeyBins = 832;            // float-like key of a score < 2^31
constexpr int kRedBins = 32;             // bins per reduce workgroup
constexpr int kSubBits = 12;
constexpr int kSubBins = 1 << kSubBits;  // second-level histogram / refinement digit
constexpr int kThrThreads = 1024;
constexpr int kMaxTilesPerSeq = 8192;    // LDS tile tables of the threshold kernel (8M positions)
constexpr int kLastMax = kThrThreads;    // entries the last digits take, one per thread
constexpr int kCandHead = 16;            // candidates per tile in the dense head array
constexpr int kListMax = 8 * kThrThreads;  // threshold: bin B1 candidates compacted into LDS
constexpr int kMaxBatch = 4096;

struct FullState {
    int E;       // eligible positions
    int Peff;    // pool size
    int tile0;   // first global tile of this sequence
    int ntiles;  // tiles of this sequence
    int T;       // take s > T ...
    int needT;   // ... plus the first needT entries with s == T
    int kb;      // first-level bin holding the Peff-th score
    int above;   // entries in higher first-level bins
};
static_assert(sizeof(FullState) == 32, "FullState size");

// Arrays of one selection target.  Target 0 ranks the pool (P_eff =
// min(P, E)); the optional target 1 ranks the top k of the same scores
// (min(k, E)), which is the top k of the pool under the same order.
struct FullTarget {
    FullState* st;        // [B]
    uint32_t* hist2;      // [B][kSubBins]
    int* tile_above;      // [Tmax] entries of the tile above bin B1
    int* tile_cnt;        // [Tmax] entries of the tile inside bin B1
    int* tile_off;        // [Tmax][2] output offsets among s > T and among s == T
    int* cand_head;       // [kCandHead][Tmax] scores of every tile's first candidates,
                          // slot-major so that one slot of consecutive tiles is contiguous
    int* cand;            // [Tmax][kTile] scores inside bin B1, per tile (slots >= kCandHead;
                          // the first kCandHead live in cand_head)
};

// The workspace as the kernels see it.  Each per-target array holds target
// 0's block, then target 1's (used when k > 0), so a target's arrays are
// these bases plus fixed strides: no kernel indexes its arguments by target.
// The sizes and the arrays the gather and threshold kernels read first come
// first: kernels that take FullWs as their first argument receive those 64
// bytes in SGPRs with the wave.
struct FullWs {
    int B;                // sequences
    int tmax;             // Tmax: tiles of the layout, the slot stride of cand_head
    int k;                // size of target 1, 0 when there is none
    int plane_tiles;      // > 0: the lists are the planes of one sequence, tile t in list
                          // t / plane_tiles (no lookup); 0: found from the lists' states
    int* scores;          // [Tmax][kTile]
    FullState* st;        // [2][B]
    uint32_t* hist2;      // [2][B][kSubBins]
    int* tile_cnt;        // [2][Tmax]
    int* tile_above;      // [2][Tmax]
    int* cand_head;       // [2][kCandHead][Tmax]
    int* tile_off;        // [2][Tmax][2]
    int* cand;            // [2][Tmax][kTile]
    uint32_t* hist;       // [B][kKeyBins]
    uint16_t* tile_hist;  // [Tmax][kKeyBins]
};

// The arrays of target y.
__device__ __forceinline__ FullTarget target(const FullWs& w, int y) {
    const size_t T = (size_t)w.tmax;
    FullTarget g;
    g.st = w.st + (size_t)y * w.B;
    g.hist2 = w.hist2 + (size_t)y * w.B * kSubBins;
    g.tile_above = w.tile_above + y * T;
    g.tile_cnt = w.tile_cnt + y * T;
    g.tile_off = w.tile_off + y * T * 2;
    g.cand_head = w.cand_head + y * T * kCandHead;
    g.cand = w.cand + y * T * kTile;
    return g;
}

// Where a target's result goes: pos (and score, when not null) [B][stride],
// ascending positions, tail -1; len [B].
struct FullOut {
    int* pos;
    int* score;
    int* len;
    int stride;
};

// Tiles of the scratch layout and of every per-tile grid: an upper bound on
// the tiles of all sequences, rounded up to a multiple of 8 so that tile t of
// every grid row lands on the same XCD (workgroup i runs on XCD i mod 8) as
// the scoring workgroup that wrote its scores.
static long long full_tile_bound(int B, long long total_len) {
    return (total_len / kTile + B + 1 + 7) / 8 * 8;
}

// Workspace of B score lists laid out over T tiles.
static size_t full_ws_layout(int B, long long T, int ntargets, char* base, FullWs* w) {
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = round_up(off + bytes, 256);
        return base ? base + at : nullptr;
    };
    const size_t n = (size_t)ntargets;
    FullWs x = {};
    x.hist = reinterpret_cast<uint32_t*>(take(4ull * B * kKeyBins));
    x.tile_hist = reinterpret_cast<uint16_t*>(take(2ull * (size_t)T * kKeyBins));
    x.scores = reinterpret_cast<int*>(take(4ull * (size_t)T * kTile));
    x.st = reinterpret_cast<FullState*>(take(n * sizeof(FullState) * (size_t)B));
    x.hist2 = reinterpret_cast<uint32_t*>(take(n * 4ull * B * kSubBins));
    x.tile_above = reinterpret_cast<int*>(take(n * 4ull * T));
    x.tile_cnt = reinterpret_cast<int*>(take(n * 4ull * T));
    x.tile_off = reinterpret_cast<int*>(take(n * 8ull * T));
    x.cand_head = reinterpret_cast<int*>(take(n * 4ull * (size_t)T * kCandHead));
    x.cand = reinterpret_cast<int*>(take(n * 4ull * (size_t)T * kTile));
    x.B = B;
    x.tmax = (int)T;
    x.k = 0;
    x.plane_tiles = 0;
    if (w) *w = x;
    return off;
}

size_t index_full_ws_bytes(int B, long long total_len, int P, int k) {
    (void)P;
    return full_ws_layout(B, full_tile_bound(B, total_len), k > 0 ? 2 : 1, nullptr, nullptr);
}

// A verify block of T tokens per sequence.  Per-token selection ranks T lists
// per sequence (list b * T + t, token t's own eligible positions); their
// tiles lie in T planes of full_tile_bound(B, total_len) tiles each, list
// (b, t) at the tiles of sequence b in plane t, so tile g of every plane sits
// on the XCD of the scoring workgroup g that wrote it.  Shared selection ranks
// one list per sequence (the best score over the block) in one plane.
static int block_planes(int T, int shared) { return shared ? 1 : T; }

size_t index_full_block_ws_bytes(int B, int T, int shared, long long total_len, int k) {
    const int planes = block_planes(T, shared);
    return full_ws_layout(B * planes, planes * full_tile_bound(B, total_len), k > 0 ? 2 : 1,
                          nullptr, nullptr);
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

// Digit of at most kSubBits bits over [lo, hi]: shift and bin count.
__device__ __forceinline__ void sub_digit(int lo, int hi, int& sh, int& nb) {
    const unsigned width = (unsigned)(hi - lo) + 1u;
    const int bits = 32 - __clz(width - 1u);
    sh = bits > kSubBits ? bits - kSubBits : 0;
    nb = (int)(((width - 1u) >> sh) + 1u);
}

// Bin holding the need-th largest entry of a histogram (bins ascending in
// value); every thread gets (bin, entries in higher bins, entries in the bin).
// Requires 1 <= need <= total count.  Thread t owns the PER consecutive bins
// starting at (NT - 1 - t) * PER, whose counts it passes in c.
template <int NT, int PER>
__device__ __forceinline__ void find_bin_counts(const int (&c)[PER], int need, int* s_tmp,
                                                int* s_res, int& bin_out, int& above_out,
                                                int& cnt_out) {
    const int r = NT - 1 - threadIdx.x;          // thread 0 owns the highest bins
    int mysum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) mysum += c[i];
    int tot;
    const int above = block_exclusive_scan<NT>(mysum, s_tmp, tot);
    if (above < need && need <= above + mysum) {
        int acc = above;
#pragma unroll
        for (int i = PER - 1; i >= 0; --i) {
            if (acc < need && need <= acc + c[i]) {
                s_res[0] = r * PER + i;
                s_res[1] = acc;
                s_res[2] = c[i];
            }
            acc += c[i];
        }
    }
    __syncthreads();
    bin_out = s_res[0];
    above_out = s_res[1];
    cnt_out = s_res[2];
    __syncthreads();
}

template <int NT, int PER, typename H>
__device__ __forceinline__ void find_bin(const H* h, int nb, int need, int* s_tmp, int* s_res,
                                         int& bin_out, int& above_out, int& cnt_out) {
    const int r = NT - 1 - threadIdx.x;
    int c[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int bin = r * PER + i;
        c[i] = bin < nb ? (int)h[bin] : 0;
    }
    find_bin_counts<NT, PER>(c, need, s_tmp, s_res, bin_out, above_out, cnt_out);
}

// Tile t -> sequence, from the lengths (up to kMaxBatch sequences, 8 per
// thread).  Returns the sequence (or -1 past the last tile) and the layout of
// that sequence.  The lists' states are written on the way (write_states):
// st0 gets P_eff = min(P, E) and st1 (when not null) min(k, E).
struct TileInfo {
    int b, tile0, E;
    long long roff;
};

__device__ __forceinline__ FullState initial_state(int E, int P, int tile0, int nt) {
    FullState s;
    s.E = E;
    s.Peff = E < P ? E : P;
    s.tile0 = tile0;
    s.ntiles = nt;
    s.T = 0x7FFFFFFF;
    s.needT = 0;
    s.kb = 0;
    s.above = 0;
    return s;
}

// States of sequence b's lists: one per plane.  The list of plane i ranks
// E - (planes - 1 - i) positions (a verify block's token i sees one position
// fewer than token i + 1) over the tiles of the sequence in plane i.  With one
// plane that is the sequence's own list.
__device__ __forceinline__ void write_state(FullState* st0, FullState* st1, int b, int E, int P,
                                            int k, int tile0, int planes, int TB, int i) {
    const int Ei = max(0, E - (planes - 1 - i));
    const int nt = (Ei + kTile - 1) / kTile;
    st0[(size_t)b * planes + i] = initial_state(Ei, P, i * TB + tile0, nt);
    if (st1) st1[(size_t)b * planes + i] = initial_state(Ei, k, i * TB + tile0, nt);
}

__device__ __forceinline__ void write_states(FullState* st0, FullState* st1, int b, int E, int P,
                                             int k, int tile0, int planes, int TB) {
    for (int i = 0; i < planes; ++i) write_state(st0, st1, b, E, P, k, tile0, planes, TB, i);
}

// One sequence: no scan, no LDS, no barrier.
__device__ __forceinline__ TileInfo map_tile_one(const int* __restrict__ len,
                                                 const long long* __restrict__ row_off,
                                                 int window, int P, int k, int t,
                                                 FullState* st0, FullState* st1, int planes = 1,
                                                 int TB = 0) {
    const int L = len[0];
    const long long roff = row_off[0];
    const int E = L > window ? L - window : 0;
    const int nt = (E + kTile - 1) / kTile;
    if (t == 0 && st0)                                   // the lists' states, a thread each
        for (int i = threadIdx.x; i < planes; i += blockDim.x)
            write_state(st0, st1, 0, E, P, k, 0, planes, TB, i);
    TileInfo r;
    r.b = t < nt ? 0 : -1;
    r.tile0 = 0;
    r.E = E;
    r.roff = roff;
    return r;
}

template <int NT>
__device__ __forceinline__ TileInfo map_tile(const int* __restrict__ len,
                                          const long long* __restrict__ row_off, int B,
                                          int window, int P, int k, int t, FullState* st0,
                                          FullState* st1, int planes = 1, int TB = 0) {
    __shared__ int s_tmp[NT / kWave];
    __shared__ int s_b, s_tile0, s_E;
    __shared__ long long s_roff;
    TileInfo r;
    constexpr int SPT = kMaxBatch / NT;                   // sequences per thread
    const int first = threadIdx.x * SPT;
    int nt[SPT], Ev[SPT];
    int sum_t = 0;
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
        const int b = first + i;
        int E = 0;
        if (b < B) {
            const int L = len[b];
            E = L > window ? L - window : 0;
        }
        Ev[i] = E;
        nt[i] = (E + kTile - 1) / kTile;
        sum_t += nt[i];
    }
    if (threadIdx.x == 0) s_b = -1;
    int tot_t;
    int pre_t = block_exclusive_scan<NT>(sum_t, s_tmp, tot_t);
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
        const int b = first + i;
        if (b < B) {
            if (t >= pre_t && t < pre_t + nt[i]) {
                s_b = b;
                s_tile0 = pre_t;
                s_E = Ev[i];
                s_roff = row_off[b];
            }
            // one list per sequence: workgroup 0 writes them all; several
            // (per-token lists) are written by the sequence's first tile,
            // spread over its threads, and workgroup 0 covers sequences
            // without tiles
            if (t == 0 && st0 && (planes == 1 || nt[i] == 0))
                write_states(st0, st1, b, Ev[i], P, k, pre_t, planes, TB);
        }
        pre_t += nt[i];
    }
    __syncthreads();
    r.b = s_b;
    r.tile0 = s_tile0;
    r.E = s_E;
    r.roff = s_roff;
    if (planes > 1 && st0 && r.b >= 0 && t == r.tile0)
        for (int i = threadIdx.x; i < planes; i += NT)
            write_state(st0, st1, r.b, r.E, P, k, r.tile0, planes, TB, i);
    return r;
}

// ---- 1. score + per-tile histogram -------------------------------------------------
// Scores go to score_out + (seq_stride < 0 ? t * kTile : b * seq_stride + p).
// Eight waves per workgroup, 128 tokens (8 groups of 16) per wave, so a CU
// holds many waves whose scoring overlaps the others' key loads.
// Load order: the index query and head weights first (with one sequence they
// need no lookup, so they travel together with the length), then all of the
// wave's key loads, and only then the first barrier, so nothing waits between
// the length arriving and the key stream starting.
// ONE: one sequence (no tile lookup).  Both instances fit six waves per SIMD
// (three workgroups per CU; the batch instance spills one key operand to
// fit), so 768 of a 1M context's 1,024 tiles run in the first round.
template <int NB, bool ONE>
__global__ __launch_bounds__(kScoreThreads, 6) void full_score_kernel(
    const int8_t* __restrict__ q, const int8_t* __restrict__ wts,
    const int8_t* __restrict__ keys, const long long* __restrict__ row_off,
    const int* __restrict__ len, int B, int H, int window, int P, FullWs w,
    int* __restrict__ score_out, long long seq_stride) {
    __shared__ uint32_t s_hist[kKeyBins];
    __shared__ __attribute__((aligned(16))) uint32_t s_w[kDk];   // head weights, one dword each
    const int t = blockIdx.x;
    const int l = lane_id();
    const int wave = threadIdx.x / kWave;
    i32x4 qa[NB];
    int wv = 0;
    auto load_query = [&](int b) {
        const int8_t* qb = q + (size_t)b * H * kDk + (l >> 4) * 16;
#pragma unroll
        for (int mb = 0; mb < NB; ++mb) {
            const int h = mb * 16 + (l & 15);
            qa[mb] = h < H ? *reinterpret_cast<const i32x4*>(qb + (size_t)h * kDk)
                           : i32x4{0, 0, 0, 0};
        }
        if (threadIdx.x < H) wv = (uint8_t)wts[(size_t)b * H + threadIdx.x];
    };
    TileInfo ti;
    if constexpr (ONE) {
        load_query(0);
        ti = map_tile_one(len, row_off, window, P, w.k, t, w.st, w.k > 0 ? w.st + B : nullptr);
        if (ti.b < 0) return;                              // past the last tile
    } else {
        ti = map_tile<kScoreThreads>(len, row_off, B, window, P, w.k, t, w.st,
                                     w.k > 0 ? w.st + B : nullptr);
        if (ti.b < 0) return;
        load_query(ti.b);
    }
    const int b = ti.b;

    const int p_tile = (t - ti.tile0) * kTile;                 // first position
    const int8_t* kbase = keys + ((size_t)ti.roff + p_tile) * kDk + (l >> 4) * 16;
    const int nvalid = min(kTile, ti.E - p_tile);
    // wave w scores tokens [128w, 128w + 128): 8 groups of 16, all loads issued
    // before the first MFMA
    constexpr int kWaves = kScoreThreads / kWave;
    constexpr int kGroups = kTile / (kWaves * 16);
    const int t0 = (kTile / kWaves) * wave;
    i32x4 kop[kGroups];
#pragma unroll
    for (int u = 0; u < kGroups; ++u) {
        int tok = t0 + 16 * u + (l & 15);
        tok = tok < nvalid ? tok : 0;
        kop[u] = *reinterpret_cast<const i32x4*>(kbase + (size_t)tok * kDk);
    }
    asm volatile("" ::: "memory");                             // keys are in flight first
    for (int i = threadIdx.x; i < kKeyBins; i += kScoreThreads) s_hist[i] = 0;
    if (threadIdx.x < kDk) s_w[threadIdx.x] = (uint32_t)wv;
    __syncthreads();                                           // histogram zeroed, weights in LDS
    // lane l weighs heads 16 mb + 4 (l >> 4) + i, i = 0..3: one 16-byte LDS
    // read per block, each weight a whole dword, so the epilogue is one
    // v_max_i32 and one v_mad_u32_u24 per product (no byte selects)
    uint32_t wr[NB][4];
#pragma unroll
    for (int mb = 0; mb < NB; ++mb) {
        const u32x4 w4 = *reinterpret_cast<const u32x4*>(s_w + 16 * mb + 4 * (l >> 4));
#pragma unroll
        for (int i = 0; i < 4; ++i) wr[mb][i] = w4[i];
    }
    int* sc_out = score_out + (seq_stride < 0 ? (size_t)t * kTile
                                              : (size_t)b * (size_t)seq_stride + p_tile);
#pragma unroll
    for (int it = 0; it < kGroups / 4; ++it) {
        if (t0 + 64 * it >= nvalid) break;                     // wave-uniform
        uint32_t part[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) part[u] = score_partial16<NB>(qa, wr, kop[4 * it + u]);
        const int mine = (int)reduce_rows4(part);              // token t0 + 64 it + l
        const int tok = t0 + 64 * it + l;
        if (tok < nvalid) {
            sc_out[tok] = mine;
            atomicAdd(&s_hist[score_key(mine)], 1u);
        }
    }
    __syncthreads();
    // per-tile histogram, u16 (a tile has <= 1,024 entries), two bins per word
    uint32_t* th = reinterpret_cast<uint32_t*>(w.tile_hist + (size_t)t * kKeyBins);
    for (int i = threadIdx.x; i < kKeyBins / 2; i += kScoreThreads)
        th[i] = s_hist[2 * i] | (s_hist[2 * i + 1] << 16);
}

// ---- 1b. score a block of T query tokens -------------------------------------------
// The same tiles and MFMA scoring, with the key operands loaded once and
// scored against many query tokens in turn: each wave holds its 128 key rows
// in registers while the tokens' queries and weights come from LDS, eight
// tokens at a time.
// planes == T (per-token lists): token t's scores of the positions it may
// rank (p < E - (T - 1 - t), E the last token's count) go to tile g of plane
// t, each plane with its own histogram; the tokens are split over grid rows
// of kBlockGroup tokens (a long block, e.g. a prefill chunk, then keeps the
// chip busy; each row reloads the tile's keys).  planes == 1 (shared list):
// one grid row; the best score over all T tokens of each position every token
// may rank (E is then the first token's count) goes to tile g.  Scores go to
// score_out in that tile layout (seq_stride < 0) or to list (b, plane) at
// (b * planes + plane) * seq_stride + p.
constexpr int kMaxBlockT = 1024;
constexpr int kBlockChunk = 8;            // tokens whose queries sit in LDS at once
constexpr int kBlockGroup = 32;           // per-token lists: tokens per grid row

// Dynamic LDS of the block kernel: queries [kBlockChunk][16 NB][64] (heads
// past H are zero), weights [kBlockChunk][64] dwords (zero past H),
// histograms [kBlockChunk or 1][kKeyBins].
static size_t block_score_lds(int NB, int planes) {
    return (size_t)kBlockChunk * NB * 16 * kDk + (size_t)kBlockChunk * 64 * 4 +
           (size_t)(planes == 1 ? 1 : kBlockChunk) * kKeyBins * 4;
}

static int block_groups(int T, int planes) {
    return planes == 1 ? 1 : (T + kBlockGroup - 1) / kBlockGroup;
}

template <int NB>
__global__ __launch_bounds__(kScoreThreads) void full_score_block_kernel(
    const int8_t* __restrict__ q, const int8_t* __restrict__ wts,
    const int8_t* __restrict__ keys, const long long* __restrict__ row_off,
    const int* __restrict__ len, int B, int H, int window, int P, FullWs w, int T, int planes,
    int TB, int* __restrict__ score_out, long long seq_stride) {
    extern __shared__ __attribute__((aligned(16))) unsigned char s_dyn[];
    i32x4* s_q = reinterpret_cast<i32x4*>(s_dyn);
    uint32_t* s_w = reinterpret_cast<uint32_t*>(s_dyn + (size_t)kBlockChunk * NB * 16 * kDk);
    uint32_t* s_hist = s_w + kBlockChunk * 64;
    const int g = blockIdx.x;
    const int l = lane_id();
    const int wave = threadIdx.x / kWave;
    // grid row 0 writes the lists' states
    FullState* st0 = blockIdx.y == 0 ? w.st : nullptr;
    FullState* st1 = blockIdx.y == 0 && w.k > 0 ? w.st + w.B : nullptr;
    const TileInfo ti = B == 1 ? map_tile_one(len, row_off, window, P, w.k, g, st0, st1, planes, TB)
                               : map_tile<kScoreThreads>(len, row_off, B, window, P, w.k, g, st0,
                                                         st1, planes, TB);
    if (ti.b < 0) return;                                      // past the last tile
    const int b = ti.b;
    const int p_tile = (g - ti.tile0) * kTile;
    const int8_t* kbase = keys + ((size_t)ti.roff + p_tile) * kDk + (l >> 4) * 16;
    const int nvalid = min(kTile, ti.E - p_tile);
    constexpr int kWaves = kScoreThreads / kWave;
    constexpr int kGroups = kTile / (kWaves * 16);
    const int t0 = (kTile / kWaves) * wave;
    i32x4 kop[kGroups];
#pragma unroll
    for (int u = 0; u < kGroups; ++u) {
        int tok = t0 + 16 * u + (l & 15);
        tok = tok < nvalid ? tok : 0;
        kop[u] = *reinterpret_cast<const i32x4*>(kbase + (size_t)tok * kDk);
    }
    asm volatile("" ::: "memory");                             // keys are in flight first
    const int tk_begin = planes == 1 ? 0 : blockIdx.y * kBlockGroup;
    const int tk_end = planes == 1 ? T : min(T, tk_begin + kBlockGroup);
    int best[kGroups / 4];
#pragma unroll
    for (int it = 0; it < kGroups / 4; ++it) best[it] = 0;
    for (int c0 = tk_begin; c0 < tk_end; c0 += kBlockChunk) {
        const int nc = min(kBlockChunk, tk_end - c0);          // uniform
        if (c0 > tk_begin) __syncthreads();                    // the last chunk's LDS is read
        {
            const int8_t* qb = q + ((size_t)b * T + c0) * H * kDk;
            const int pieces = nc * NB * 16 * 4;               // 16-byte pieces, zero past H
            for (int i = threadIdx.x; i < pieces; i += kScoreThreads) {
                const int tk = i / (NB * 64), h = (i >> 2) % (NB * 16);
                s_q[i] = h < H ? *reinterpret_cast<const i32x4*>(qb + ((size_t)tk * H + h) * kDk +
                                                                 (i & 3) * 16)
                               : i32x4{0, 0, 0, 0};
            }
            for (int i = threadIdx.x; i < nc * 64; i += kScoreThreads) {
                const int tk = i >> 6, h = i & 63;
                s_w[i] = h < H ? (uint32_t)(uint8_t)wts[((size_t)b * T + c0 + tk) * H + h] : 0u;
            }
            if (planes > 1 || c0 == 0)
                for (int i = threadIdx.x; i < (planes == 1 ? 1 : nc) * kKeyBins; i += kScoreThreads)
                    s_hist[i] = 0;
        }
        __syncthreads();
        for (int tc = 0; tc < nc; ++tc) {
            const int tk = c0 + tc;                            // the token of the block
            i32x4 qa[NB];
            uint32_t wr[NB][4];
#pragma unroll
            for (int mb = 0; mb < NB; ++mb) {
                qa[mb] = s_q[((tc * NB + mb) * 16 + (l & 15)) * 4 + (l >> 4)];
                const u32x4 w4 =
                    *reinterpret_cast<const u32x4*>(s_w + tc * 64 + 16 * mb + 4 * (l >> 4));
#pragma unroll
                for (int i = 0; i < 4; ++i) wr[mb][i] = w4[i];
            }
            // per-token lists: this token's plane and its own count of positions
            const int nv = planes == 1 ? nvalid : min(kTile, ti.E - (T - 1 - tk) - p_tile);
            int* sc_out = seq_stride < 0
                              ? score_out + (size_t)(planes == 1 ? g : tk * TB + g) * kTile
                              : score_out + ((size_t)b * planes + (planes == 1 ? 0 : tk)) *
                                                (size_t)seq_stride + p_tile;
            uint32_t* hist = s_hist + (planes == 1 ? 0 : tc * kKeyBins);
#pragma unroll
            for (int it = 0; it < kGroups / 4; ++it) {
                if (t0 + 64 * it >= nvalid) break;             // wave-uniform
                uint32_t part[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) part[u] = score_partial16<NB>(qa, wr, kop[4 * it + u]);
                const int mine = (int)reduce_rows4(part);      // token t0 + 64 it + l
                const int pos = t0 + 64 * it + l;
                if (planes == 1) {
                    best[it] = tk == 0 ? mine : max(best[it], mine);
                } else if (pos < nv) {
                    sc_out[pos] = mine;
                    atomicAdd(&hist[score_key(mine)], 1u);
                }
            }
        }
        if (planes > 1) {
            __syncthreads();
            // per-tile histograms of the chunk's planes whose list reaches this tile
            for (int tc = 0; tc < nc; ++tc) {
                const int tk = c0 + tc;
                if (ti.E - (T - 1 - tk) <= p_tile) continue;   // uniform
                uint32_t* th =
                    reinterpret_cast<uint32_t*>(w.tile_hist + (size_t)(tk * TB + g) * kKeyBins);
                const uint32_t* sh = s_hist + tc * kKeyBins;
                for (int i = threadIdx.x; i < kKeyBins / 2; i += kScoreThreads)
                    th[i] = sh[2 * i] | (sh[2 * i + 1] << 16);
            }
        }
    }
    if (planes == 1) {
        int* sc_out = seq_stride < 0 ? score_out + (size_t)g * kTile
                                     : score_out + (size_t)b * seq_stride + p_tile;
#pragma unroll
        for (int it = 0; it < kGroups / 4; ++it) {
            const int pos = t0 + 64 * it + l;
            if (pos < nvalid) {
                sc_out[pos] = best[it];
                atomicAdd(&s_hist[score_key(best[it])], 1u);
            }
        }
        __syncthreads();
        uint32_t* th = reinterpret_cast<uint32_t*>(w.tile_hist + (size_t)g * kKeyBins);
        for (int i = threadIdx.x; i < kKeyBins / 2; i += kScoreThreads)
            th[i] = s_hist[2 * i] | (s_hist[2 * i + 1] << 16);
    }
}

// ---- 2. reduce the per-tile histograms ---------------------------------------------
// workgroup (c, b): bins [32c, 32c + 32) of sequence b; thread (r, k) sums
// bins 8k .. 8k+7 over tiles r, r + 64, ...
__global__ __launch_bounds__(kScanThreads) void full_reduce_kernel(FullWs w) {
    __shared__ uint32_t s_part[kScanThreads / 4][kRedBins + 1];
    const int c = blockIdx.x, b = blockIdx.y;
    const FullState st = w.st[b];                              // tile0, ntiles: both targets
    const int z = c * kScanThreads + threadIdx.x;              // clear the sub-bin histograms
    if (z < kSubBins) {
        w.hist2[(size_t)b * kSubBins + z] = 0;
        if (w.k > 0) w.hist2[((size_t)w.B + b) * kSubBins + z] = 0;
    }
    const int r = threadIdx.x >> 2, k = threadIdx.x & 3;
    uint32_t acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    constexpr int U = 8;
    for (int base = 0; base < st.ntiles; base += 64 * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tile = base + r + 64 * u;
            v[u] = tile < st.ntiles
                       ? *reinterpret_cast<const u32x4*>(w.tile_hist +
                                                         (size_t)(st.tile0 + tile) * kKeyBins +
                                                         kRedBins * c + 8 * k)
                       : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] += v[u][i] & 0xFFFFu;
                acc[2 * i + 1] += v[u][i] >> 16;
            }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) s_part[r][8 * k + i] = acc[i];
    __syncthreads();
    if (threadIdx.x < kRedBins) {
        uint32_t s = 0;
        for (int i = 0; i < kScanThreads / 4; ++i) s += s_part[i][threadIdx.x];
        w.hist[(size_t)b * kKeyBins + kRedBins * c + threadIdx.x] = s;
    }
}

// Sequence owning global tile t, from the per-sequence state (result in LDS).
__device__ int tile_seq(const FullState* __restrict__ st, int B, int t, int* s_b) {
    if (threadIdx.x == 0) *s_b = -1;
    __syncthreads();
    for (int b = threadIdx.x; b < B; b += blockDim.x) {
        const int t0 = st[b].tile0;
        if (t >= t0 && t < t0 + st[b].ntiles) *s_b = b;
    }
    __syncthreads();
    return *s_b;
}

// List of global tile t (-1 past the list's last tile) and its state.  With
// one list, or with the per-token lists of one sequence (each in its own
// plane of plane_tiles tiles), that is a single load; a batch looks the tile
// up first.
__device__ __forceinline__ int tile_state(const FullState* __restrict__ sts, int B, int t, int* s_b,
                                          FullState& st, int plane_tiles) {
    if (B == 1) {
        st = sts[0];                                  // tile0 == 0
        return t < st.ntiles ? 0 : -1;
    }
    if (plane_tiles > 0) {
        const int b = t / plane_tiles;
        st = sts[b];
        return t - st.tile0 < st.ntiles ? b : -1;
    }
    const int b = tile_seq(sts, B, t, s_b);
    if (b >= 0) st = sts[b];
    return b;
}

// ---- 3. gather: entries above / inside bin B1 --------------------------------------
// Workgroup x handles tiles G x .. G x + G - 1 (G > 1 when there are many
// tiles: every tile's scores are loaded at once, and consecutive tiles of one
// list share the bin search).
template <int G>
__global__ __launch_bounds__(kScanThreads) void full_gather_kernel(FullWs w) {
    const int B = w.B;
    __shared__ int s_b;
    __shared__ int s_tmp[kScanThreads / kWave];
    __shared__ int s_res[3];
    const int tfirst = blockIdx.x * G;
    constexpr int PER = kTile / kScanThreads;   // contiguous positions per thread
    const int i0 = threadIdx.x * PER;
    // the tiles' scores sit at t * kTile whatever their list: load them first
    int v[G][PER];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const int* sc = w.scores + (size_t)min(tfirst + i, w.tmax - 1) * kTile;
#pragma unroll
        for (int j = 0; j < PER; ++j) v[i][j] = sc[i0 + j];
    }
    const FullTarget g = target(w, blockIdx.y);
    int bprev = -1, kb = 0, above = 0, cnt = 0;
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const int t = tfirst + i;
        if (t >= w.tmax) break;                      // uniform
        FullState st;
        const int b = tile_state(g.st, B, t, &s_b, st, w.plane_tiles);
        if (b < 0) continue;                         // uniform
        const int p_tile = (t - st.tile0) * kTile;
        const int nvalid = min(kTile, st.E - p_tile);
#pragma unroll
        for (int j = 0; j < PER; ++j)
            if (i0 + j >= nvalid) v[i][j] = -1;
        if (b != bprev) {                            // uniform
            find_bin<kScanThreads, (kKeyBins + kScanThreads - 1) / kScanThreads>(
                w.hist + (size_t)b * kKeyBins, kKeyBins, st.Peff, s_tmp, s_res, kb, above, cnt);
            bprev = b;
        }
        int lo, hi, sh, nb;
        key_interval(kb, lo, hi);
        sub_digit(lo, hi, sh, nb);
        // per-thread counts of entries above / inside the bin, packed in one scan
        int n_above = 0, n_in = 0;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            n_above += v[i][j] > hi;
            n_in += v[i][j] >= lo && v[i][j] <= hi;
        }
        int tot;
        int slot = block_exclusive_scan<kScanThreads>((n_in << 16) | n_above, s_tmp, tot) >> 16;
        if (threadIdx.x == 0) {
            g.tile_above[t] = tot & 0xFFFF;
            g.tile_cnt[t] = tot >> 16;
            if (t == st.tile0) {
                g.st[b].kb = kb;
                g.st[b].above = above;
            }
        }
        int* head = g.cand_head + t;
        int* out = g.cand + (size_t)t * kTile;
        uint32_t* h2 = g.hist2 + (size_t)b * kSubBins;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            if (v[i][j] >= lo && v[i][j] <= hi) {
                if (slot < kCandHead) head[(size_t)slot * w.tmax] = v[i][j];
                else out[slot] = v[i][j];
                ++slot;
                atomicAdd(&h2[(unsigned)(v[i][j] - lo) >> sh], 1u);
            }
        }
    }
}

// ---- 4. threshold: exact select among the candidates, tile offsets ---------------
// One workgroup per sequence and target.  Tile i belongs to thread i mod 1,024
// (round u = i / 1,024).  Every thread loads its first tile's counts and the
// tile's first kCandHead candidates (dense across tiles, so the threads' loads
// are contiguous) with the sub-histogram.  All candidates of bin B1 are then
// compacted into one list in LDS (value and tile): first every thread's
// registers, then the rest (a tile with more than kCandHead, every tile of
// later rounds) in tile order, where thread t takes entries t, t + 1,024, ...
// and finds their tile by binary search over the per-tile starts.  Every
// later pass reads the list, each thread a share of the same size however the
// candidates cluster.  A list longer than kListMax is not built: the passes
// then read the registers and global memory, each thread walking its tiles.
template <bool ONE>   // ONE: a single sequence, whose first tile is 0
__global__ __launch_bounds__(kThrThreads) void full_threshold_kernel(FullWs w) {
    constexpr int NT = kThrThreads;
    constexpr int HPT = kSubBins / NT;               // sub-bins per thread
    constexpr int kCandReg = kCandHead;              // candidates of the first tile in registers
    constexpr int LPT = kListMax / NT;               // list entries per thread at most
    __shared__ uint32_t s_hist[kSubBins];
    __shared__ int s_tmp[2 * NT / kWave];
    __shared__ int s_res[4];
    __shared__ int s_val[kLastMax];                  // the last entries: scores ...
    __shared__ uint16_t s_valt[kLastMax];            // ... and their tiles
    __shared__ int s_tile[kMaxTilesPerSeq];          // list start of each tile's rest, then
                                                     // per tile: candidates > T | == T << 16
    __shared__ uint64_t s_list[kListMax];            // the list: score | tile << 32
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const FullTarget g = target(w, blockIdx.y);
    // round trip 1: the first tile's counts (needed first: loads complete in
    // order), its first candidates, the second-level histogram and the state.
    // Every load is unconditional (a thread past the last tile reads another
    // tile and then counts nothing), so none of them waits for another; with
    // one sequence (first tile 0) they need not wait for the state either
    const FullState st = g.st[b];
    const size_t tile0 = ONE ? (size_t)min(tid, w.tmax - 1)
                             : (size_t)st.tile0 + (tid < st.ntiles ? tid : 0);
    const int tc0 = g.tile_cnt[tile0];               // read for another tile too, then masked
    const int ta0 = g.tile_above[tile0];
    // slot j of consecutive tiles is contiguous: each load is coalesced
    int cr[kCandReg];                                // slots past tc0 hold stale data, unused
#pragma unroll
    for (int j = 0; j < kCandReg; ++j) cr[j] = g.cand_head[(size_t)j * w.tmax + tile0];
    int h2[HPT];
#pragma unroll
    for (int i = 0; i < HPT; ++i)
        h2[i] = (int)g.hist2[(size_t)b * kSubBins + (NT - 1 - tid) * HPT + i];
    if (st.Peff == 0) {                              // uniform
        // an empty use of the loads on this path too keeps the compiler from
        // moving them below the branch, behind the state's round trip
        int x = tc0 ^ ta0;
#pragma unroll
        for (int j = 0; j < kCandReg; ++j) x ^= cr[j];
#pragma unroll
        for (int i = 0; i < HPT; ++i) x ^= h2[i];
        asm volatile("" ::"v"(x));
        return;
    }
    const bool has0 = tid < st.ntiles;
    const int ncr = has0 ? min(tc0, kCandReg) : 0;   // candidates held in cr
    const int rounds = (st.ntiles + NT - 1) / NT;    // uniform

    // list layout: the registers' candidates in thread order, then the rest
    int reg_pre, rest_pre, nreg, nrest;
    block_exclusive_scan2<NT>(ncr, has0 ? tc0 - ncr : 0, s_tmp, reg_pre, rest_pre, nreg, nrest);
    if (has0) s_tile[tid] = rest_pre;
    for (int u = 1; u < rounds; ++u) {               // uniform; later rounds: all in the rest
        const int i = tid + u * NT;
        const int m = i < st.ntiles ? g.tile_cnt[st.tile0 + i] : 0;
        int tot;
        const int pre = block_exclusive_scan<NT>(m, s_tmp, tot);
        if (i < st.ntiles) s_tile[i] = nrest + pre;
        nrest += tot;
    }
    const int nlist = nreg + nrest;                  // uniform
    const bool inlds = nlist <= kListMax;            // uniform
    if (inlds) {
#pragma unroll
        for (int j = 0; j < kCandReg; ++j)
            if (j < ncr) s_list[reg_pre + j] = (uint32_t)cr[j] | (uint64_t)tid << 32;
    }
    __syncthreads();                                 // the rest's starts are complete
    if (inlds && nrest > 0) {                        // uniform
        const int R = (nrest + NT - 1) / NT;         // uniform, <= LPT
        int fi[LPT];                                 // last tile whose start <= entry
#pragma unroll
        for (int r = 0; r < LPT; ++r) fi[r] = 0;
        for (int step = 1 << (31 - __clz(st.ntiles)); step > 0; step >>= 1) {
#pragma unroll
            for (int r = 0; r < LPT; ++r) {
                if (r < R) {
                    const int q = min(fi[r] + step, st.ntiles - 1);
                    if (s_tile[q] <= tid + r * NT) fi[r] = q;
                }
            }
        }
        int fv[LPT];
#pragma unroll
        for (int r = 0; r < LPT; ++r) {
            const int c = tid + r * NT;
            if (r < R && c < nrest) {
                const int i = fi[r];
                const int slot = c - s_tile[i] + (i < NT ? kCandReg : 0);
                const size_t t = (size_t)st.tile0 + i;
                fv[r] = slot < kCandHead ? g.cand_head[(size_t)slot * w.tmax + t]
                                         : g.cand[t * kTile + slot];
            }
        }
#pragma unroll
        for (int r = 0; r < LPT; ++r) {
            const int c = tid + r * NT;
            if (r < R && c < nrest) s_list[nreg + c] = (uint32_t)fv[r] | (uint64_t)fi[r] << 32;
        }
    }
    __syncthreads();                                 // list complete, starts no longer needed
    for (int i = tid; i < st.ntiles; i += NT) s_tile[i] = 0;
    // without the list: fn(score) for every candidate of this thread's tile in
    // round u that is not held in cr, read from global memory
    auto visit_mem = [&](int u, auto&& fn) {
        const int i = tid + u * NT;
        if (i >= st.ntiles) return;
        const size_t t = (size_t)st.tile0 + i;
        const int* cg = g.cand + t * kTile;
        if (u == 0) {
            for (int j = kCandReg; j < tc0; ++j) fn(cg[j]);
        } else {
            const int tc = g.tile_cnt[t];
            for (int j = 0; j < tc; ++j) fn(j < kCandHead ? g.cand_head[(size_t)j * w.tmax + t] : cg[j]);
        }
    };
    // fn(score, tile) for every candidate of the sequence, each once
    const int RL = (nlist + NT - 1) / NT;            // uniform
    auto visit_all = [&](auto&& fn) {
        if (inlds) {
            for (int r = 0; r < RL; ++r) {
                const int c = tid + r * NT;
                if (c < nlist) {
                    const uint64_t e = s_list[c];
                    fn((int)(uint32_t)e, (int)(e >> 32));
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < kCandReg; ++j)
                if (j < ncr) fn(cr[j], tid);
            for (int u = 0; u < rounds; ++u) visit_mem(u, [&](int c) { fn(c, tid + u * NT); });
        }
    };

    int lo, hi, sh, nb;
    key_interval(st.kb, lo, hi);
    sub_digit(lo, hi, sh, nb);
    int need = st.Peff - st.above;
    int d, a, cnt;
    find_bin_counts<NT, HPT>(h2, need, s_tmp, s_res, d, a, cnt);   // sub-bins >= nb hold 0
    need -= a;
    {
        const int nlo = lo + (d << sh);
        hi = sub_range_hi(nlo, sh, hi);
        lo = nlo;
    }
    // more 12-bit passes while the sub-bin holds several values and > kLastMax entries
    while (lo < hi && cnt > kLastMax) {              // uniform: lo, hi, cnt from LDS
        int sh2, nb2;
        sub_digit(lo, hi, sh2, nb2);
        for (int i = tid; i < nb2; i += NT) s_hist[i] = 0;
        __syncthreads();
        visit_all([&](int c, int) {
            if (c >= lo && c <= hi) atomicAdd(&s_hist[(unsigned)(c - lo) >> sh2], 1u);
        });
        __syncthreads();
        find_bin<NT, kSubBins / NT>(s_hist, nb2, need, s_tmp, s_res, d, a, cnt);
        need -= a;
        const int nlo = lo + (d << sh2);
        hi = sub_range_hi(nlo, sh2, hi);
        lo = nlo;
    }
    // T lies in [lo, hi]: one pass counts, per tile, the candidates above hi
    // (all > T); those in [lo, hi] are the ties at T when lo == hi, else (<=
    // kLastMax of them) they are gathered with their tiles, one per thread, the
    // last digits narrow them to T, and each thread adds its entry to its
    // tile's counts.  Ties at T are taken in position order by the write kernel.
    if (tid == 0) s_res[3] = 0;
    __syncthreads();
    const bool single = lo == hi;                    // uniform
    visit_all([&](int c, int i) {
        uint32_t* ti = reinterpret_cast<uint32_t*>(&s_tile[i]);
        if (c > hi) {
            atomicAdd(ti, 1u);
        } else if (c >= lo) {
            if (single) {
                atomicAdd(ti, 0x10000u);
            } else {
                const int slot = atomicAdd(&s_res[3], 1);
                if (slot < kLastMax) {
                    s_val[slot] = c;
                    s_valt[slot] = (uint16_t)i;
                }
            }
        }
    });
    __syncthreads();
    if (!single) {
        const int x = tid < cnt ? s_val[tid] : -1;
        const int xt = tid < cnt ? (int)s_valt[tid] : 0;
        narrow_to_value(x, lo, hi, need, cnt, s_hist, s_res);   // lo = hi = T
        if (x >= lo) atomicAdd(reinterpret_cast<uint32_t*>(&s_tile[xt]), x > lo ? 1u : 0x10000u);
    }
    const int T = lo, needT = need;
    __syncthreads();

    // per tile: entries above T (above bin B1 or candidates > T) and at T; exclusive
    // prefix over this sequence's tiles, in tile order
    int og = 0, oe = 0;
    for (int u = 0; u < rounds; ++u) {               // uniform
        const int i = tid + u * NT;
        int gl = 0, el = 0;
        if (i < st.ntiles) {
            const int x = s_tile[i];
            gl = (u == 0 ? ta0 : g.tile_above[st.tile0 + i]) + (x & 0xFFFF);
            el = (int)((unsigned)x >> 16);
        }
        int pg, pe, tg, te;
        block_exclusive_scan2<NT>(gl, el, s_tmp, pg, pe, tg, te);
        if (i < st.ntiles) {
            g.tile_off[2 * (st.tile0 + i)] = og + pg;
            g.tile_off[2 * (st.tile0 + i) + 1] = oe + pe;
        }
        og += tg;
        oe += te;
    }
    if (tid == 0) {
        g.st[b].T = T;
        g.st[b].needT = needT;
    }
}

// ---- 5. write: ordered compaction of the pool (and of the top k) -----------------
// blockIdx.y selects the target and its output.  Workgroup x handles tiles
// G x .. G x + G - 1, and fills the tails of the lists with those indices.
template <int G>
__global__ __launch_bounds__(kScanThreads) void full_write_kernel(FullWs w, FullOut o0,
                                                                  FullOut o1) {
    const int B = w.B;
    __shared__ int s_b;
    __shared__ int s_tmp[kScanThreads / kWave];
    const int tfirst = blockIdx.x * G;
    const FullTarget g = target(w, blockIdx.y);
    const FullOut o = blockIdx.y ? o1 : o0;
    constexpr int PER = kTile / kScanThreads;   // contiguous positions per thread
    const int i0 = threadIdx.x * PER;
    // the tiles' scores and output offsets sit at t whatever their list: load first
    int v[G][PER];
    int tile_gt[G], tile_eq[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const int tc = min(tfirst + i, w.tmax - 1);
        const int* sc = w.scores + (size_t)tc * kTile;
#pragma unroll
        for (int j = 0; j < PER; ++j) v[i][j] = sc[i0 + j];
        tile_gt[i] = g.tile_off[2 * tc];
        tile_eq[i] = g.tile_off[2 * tc + 1];
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const int t = tfirst + i;
        if (t >= w.tmax && t >= B) break;            // uniform
        FullState st;
        const int b = t < w.tmax ? tile_state(g.st, B, t, &s_b, st, w.plane_tiles) : -1;
        // tail fill of list t (each tile index fills at most one list's tail)
        if (t < B) {
            const int Peff = B == 1 ? g.st[0].Peff : g.st[t].Peff;
            for (int r = Peff + threadIdx.x; r < o.stride; r += kScanThreads) {
                o.pos[(size_t)t * o.stride + r] = -1;
                if (o.score) o.score[(size_t)t * o.stride + r] = -1;
            }
            if (threadIdx.x == 0) o.len[t] = Peff;
        }
        if (b < 0) continue;                         // uniform
        const int p_tile = (t - st.tile0) * kTile;
        const int nvalid = min(kTile, st.E - p_tile);
        int n_eq = 0;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            if (i0 + j >= nvalid) v[i][j] = -1;      // scores are >= 0
            n_eq += (v[i][j] >= 0) & (v[i][j] == st.T);
        }
        int tot;
        const int eq_before = block_exclusive_scan<kScanThreads>(n_eq, s_tmp, tot) + tile_eq[i];
        int n_sel = 0, eq_rank = eq_before;
        bool take[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            bool tk = false;
            if (v[i][j] < 0) tk = false;
            else if (v[i][j] > st.T) tk = true;
            else if (v[i][j] == st.T) {
                tk = eq_rank < st.needT;
                ++eq_rank;
            }
            take[j] = tk;
            n_sel += tk;
        }
        int base = tile_gt[i] + (tile_eq[i] < st.needT ? tile_eq[i] : st.needT);
        base += block_exclusive_scan<kScanThreads>(n_sel, s_tmp, tot);
        int* out_p = o.pos + (size_t)b * o.stride;
        int* out_s = o.score ? o.score + (size_t)b * o.stride : nullptr;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            if (take[j]) {
                if (base < st.Peff) {            // always true for consistent inputs
                    out_p[base] = p_tile + i0 + j;
                    if (out_s) out_s[base] = v[i][j];
                }
                ++base;
            }
        }
    }
}

// Argument checks shared by the two entry points; CSA2_OK or an error code.
static int check_scan_args(const char* fn, const signed char* q, const signed char* w,
                           const signed char* keys, const long long* row_off, const int* len,
                           int B, long long max_len, long long total_len, int H, int Dk,
                           int window) {
    if (B < 0 || max_len < 0 || total_len < 0)
        return fail(CSA2_ERR_INVALID, "%s: negative size", fn);
    if (B > kMaxBatch) return fail(CSA2_ERR_UNSUPPORTED, "%s: B > %d", fn, kMaxBatch);
    if (B == 0) return CSA2_OK;
    if (!q || !w || !keys || !row_off || !len)
        return fail(CSA2_ERR_INVALID, "%s: null pointer", fn);
    if (Dk != kDk) return fail(CSA2_ERR_UNSUPPORTED, "%s: Dk must be 64", fn);
    if (H < 1 || H > 64) return fail(CSA2_ERR_INVALID, "%s: H must be in [1, 64]", fn);
    if (window < 0) return fail(CSA2_ERR_INVALID, "%s: window < 0", fn);
    if (max_len > (long long)kMaxTilesPerSeq * kTile)
        return fail(CSA2_ERR_UNSUPPORTED, "%s: max_len > %lld", fn,
                    (long long)kMaxTilesPerSeq * kTile);
    if (!aligned(q, 16) || !aligned(keys, 16) || !aligned(row_off, 8) || !aligned(len, 4))
        return fail(CSA2_ERR_INVALID, "%s: misaligned pointer", fn);
    return CSA2_OK;
}

static int launch_score(int H, unsigned tiles, hipStream_t s, const signed char* q,
                        const signed char* w, const signed char* keys, const long long* row_off,
                        const int* len, int B, int window, int P, const FullWs& fw, int* out,
                        long long seq_stride) {
    const int8_t* q8 = reinterpret_cast<const int8_t*>(q);
    const int8_t* w8 = reinterpret_cast<const int8_t*>(w);
    const int8_t* k8 = reinterpret_cast<const int8_t*>(keys);
    const dim3 grid(tiles), blk(kScoreThreads);
    auto launch = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, grid, blk, 0, s, q8, w8, k8, row_off, len, B, H, window, P, fw,
                           out, seq_stride);
    };
    const bool one = B == 1;
    switch ((H + 15) / 16) {
        case 1: one ? launch(full_score_kernel<1, true>) : launch(full_score_kernel<1, false>); break;
        case 2: one ? launch(full_score_kernel<2, true>) : launch(full_score_kernel<2, false>); break;
        case 3: one ? launch(full_score_kernel<3, true>) : launch(full_score_kernel<3, false>); break;
        default: one ? launch(full_score_kernel<4, true>) : launch(full_score_kernel<4, false>); break;
    }
    return launch_status("full_score");
}

static int launch_score_block(int H, int T, int shared, unsigned TB, hipStream_t s,
                              const signed char* q, const signed char* w, const signed char* keys,
                              const long long* row_off, const int* len, int B, int window, int P,
                              const FullWs& fw, int* out, long long seq_stride) {
    const int planes = block_planes(T, shared);
    // per-token lists: tiles over the last token's positions (it sees the
    // most); shared list: over the first token's, the ones every token sees
    const int win = shared ? window + T - 1 : window;
    const int8_t* q8 = reinterpret_cast<const int8_t*>(q);
    const int8_t* w8 = reinterpret_cast<const int8_t*>(w);
    const int8_t* k8 = reinterpret_cast<const int8_t*>(keys);
    const dim3 grid(TB, block_groups(T, planes)), blk(kScoreThreads);
    const int NB = (H + 15) / 16;
    const size_t lds = block_score_lds(NB, planes);
    const int tb = (int)TB;
    switch (NB) {
        case 1: hipLaunchKernelGGL(full_score_block_kernel<1>, grid, blk, lds, s, q8, w8, k8, row_off, len, B, H, win, P, fw, T, planes, tb, out, seq_stride); break;
        case 2: hipLaunchKernelGGL(full_score_block_kernel<2>, grid, blk, lds, s, q8, w8, k8, row_off, len, B, H, win, P, fw, T, planes, tb, out, seq_stride); break;
        case 3: hipLaunchKernelGGL(full_score_block_kernel<3>, grid, blk, lds, s, q8, w8, k8, row_off, len, B, H, win, P, fw, T, planes, tb, out, seq_stride); break;
        default: hipLaunchKernelGGL(full_score_block_kernel<4>, grid, blk, lds, s, q8, w8, k8, row_off, len, B, H, win, P, fw, T, planes, tb, out, seq_stride); break;
    }
    return launch_status("full_score_block");
}

// Checks of the verify-block arguments: CSA2_OK or an error code.
static int check_block_args(const char* fn, int B, int T, int shared, int window) {
    if (T < 1 || shared < 0 || shared > 1)
        return fail(CSA2_ERR_INVALID, "%s: T < 1 or shared not 0/1", fn);
    if (T > kMaxBlockT) return fail(CSA2_ERR_UNSUPPORTED, "%s: T > %d", fn, kMaxBlockT);
    if (window > (1 << 30)) return fail(CSA2_ERR_UNSUPPORTED, "%s: window > 2^30", fn);
    if ((long long)B * block_planes(T, shared) > 65535)
        return fail(CSA2_ERR_UNSUPPORTED, "%s: more than 65535 lists", fn);
    return CSA2_OK;
}

// Kernels 2-5 over the lists of fw (fw.B lists, `tiles` tiles), whose
// scores, per-tile histograms and initial states kernel 1 has written.
static int launch_chain(const FullWs& fw, unsigned tiles, int P, int k, int* pool_pos,
                        int* pool_score, int* pool_len, int* sel_pos, int* sel_len,
                        hipStream_t s, const char* fn) {
    const int ntg = k > 0 ? 2 : 1;
    const int nl = fw.B;
    const dim3 blk(kScanThreads);
    // very many tiles (the per-token lists of a prompt chunk): four per gather
    // and write workgroup, so each workgroup keeps four tiles' loads in flight
    // (prefill_128k_chunk256: index call 434 -> 418 us); with a few thousand
    // tiles one per workgroup is faster (ragged32_1m, ctx_1m_block5: 3-4 us)
    const bool many = tiles > 16384;
    hipLaunchKernelGGL(full_reduce_kernel, dim3(kKeyBins / kRedBins, nl), blk, 0, s, fw);
    if (many)
        hipLaunchKernelGGL(full_gather_kernel<4>, dim3((tiles + 3) / 4, ntg), blk, 0, s, fw);
    else
        hipLaunchKernelGGL(full_gather_kernel<1>, dim3(tiles, ntg), blk, 0, s, fw);
    if (nl == 1)
        hipLaunchKernelGGL(full_threshold_kernel<true>, dim3(nl, ntg), dim3(kThrThreads), 0, s, fw);
    else
        hipLaunchKernelGGL(full_threshold_kernel<false>, dim3(nl, ntg), dim3(kThrThreads), 0, s, fw);
    const unsigned wgrid = tiles > (unsigned)nl ? tiles : (unsigned)nl;
    const FullOut o0 = {pool_pos, pool_score, pool_len, P};
    const FullOut o1 = {sel_pos, nullptr, sel_len, k};
    if (many)
        hipLaunchKernelGGL(full_write_kernel<4>, dim3((wgrid + 3) / 4, ntg), blk, 0, s, fw, o0, o1);
    else
        hipLaunchKernelGGL(full_write_kernel<1>, dim3(wgrid, ntg), blk, 0, s, fw, o0, o1);
    return launch_status(fn);
}

// Checks of the pool and selection arguments shared by the Full entry points.
static int check_pool_args(const char* fn, int P, int k, const int* pool_pos,
                           const int* pool_score, const int* pool_len, const int* sel_pos,
                           const int* sel_len) {
    if (P < 1) return fail(CSA2_ERR_INVALID, "%s: P < 1", fn);
    if (k < 0 || k > P) return fail(CSA2_ERR_INVALID, "%s: k must be in [0, P]", fn);
    if (!pool_pos || !pool_score || !pool_len || (k > 0 && (!sel_pos || !sel_len)))
        return fail(CSA2_ERR_INVALID, "%s: null pointer", fn);
    return CSA2_OK;
}

}  // namespace csa2

using namespace csa2;

extern "C" int csa2_index_full(const signed char* q, const signed char* w,
                               const signed char* keys, const long long* row_off,
                               const int* len, int B, long long max_len, long long total_len,
                               int H, int Dk, int window, int P, int* pool_pos,
                               int* pool_score, int* pool_len, int k, int* sel_pos,
                               int* sel_len, void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "csa2_index_full";
    if (int e = check_scan_args(fn, q, w, keys, row_off, len, B, max_len, total_len, H, Dk,
                                window))
        return e;
    if (B == 0) return CSA2_OK;
    if (int e = check_pool_args(fn, P, k, pool_pos, pool_score, pool_len, sel_pos, sel_len))
        return e;
    const size_t need = index_full_ws_bytes(B, total_len, P, k);
    if (!ws || ws_bytes < need || !aligned(ws, 256))
        return fail(CSA2_ERR_WORKSPACE, "%s: workspace needs %zu bytes (256-aligned)", fn, need);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const long long tiles = full_tile_bound(B, total_len);
    FullWs fw;
    full_ws_layout(B, tiles, k > 0 ? 2 : 1, reinterpret_cast<char*>(ws), &fw);
    fw.k = k;
    if (int e = launch_score(H, (unsigned)tiles, s, q, w, keys, row_off, len, B, window, P, fw,
                             fw.scores, -1))
        return e;
    return launch_chain(fw, (unsigned)tiles, P, k, pool_pos, pool_score, pool_len, sel_pos,
                        sel_len, s, "csa2_index_full launch");
}

extern "C" int csa2_index_full_block(const signed char* q, const signed char* w,
                                     const signed char* keys, const long long* row_off,
                                     const int* len, int B, int T, int shared, long long max_len,
                                     long long total_len, int H, int Dk, int window, int P,
                                     int* pool_pos, int* pool_score, int* pool_len, int k,
                                     int* sel_pos, int* sel_len, void* ws, size_t ws_bytes,
                                     void* stream) {
    const char* fn = "csa2_index_full_block";
    if (int e = check_scan_args(fn, q, w, keys, row_off, len, B, max_len, total_len, H, Dk,
                                window))
        return e;
    if (int e = check_block_args(fn, B, T, shared, window)) return e;
    if (B == 0) return CSA2_OK;
    if (int e = check_pool_args(fn, P, k, pool_pos, pool_score, pool_len, sel_pos, sel_len))
        return e;
    const int planes = block_planes(T, shared);
    const size_t need = index_full_block_ws_bytes(B, T, shared, total_len, k);
    if (!ws || ws_bytes < need || !aligned(ws, 256))
        return fail(CSA2_ERR_WORKSPACE, "%s: workspace needs %zu bytes (256-aligned)", fn, need);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const long long TB = full_tile_bound(B, total_len);
    FullWs fw;
    full_ws_layout(B * planes, planes * TB, k > 0 ? 2 : 1, reinterpret_cast<char*>(ws), &fw);
    fw.k = k;
    if (B == 1 && planes > 1) fw.plane_tiles = (int)TB;     // list v owns plane v
    // per-token lists: tiles over the last token's positions (it sees the
    // most); shared list: over the first token's, the ones every token sees
    if (int e = launch_score_block(H, T, shared, (unsigned)TB, s, q, w, keys, row_off, len, B,
                                   window, P, fw, fw.scores, -1))
        return e;
    return launch_chain(fw, (unsigned)(planes * TB), P, k, pool_pos, pool_score, pool_len,
                        sel_pos, sel_len, s, "csa2_index_full_block launch");
}

extern "C" int csa2_index_score(const signed char* q, const signed char* w,
                                const signed char* keys, const long long* row_off,
                                const int* len, int B, long long max_len, long long total_len,
                                int H, int Dk, int window, int* score, void* ws, size_t ws_bytes,
                                void* stream) {
    if (int e = check_scan_args("csa2_index_score", q, w, keys, row_off, len, B, max_len,
                                total_len, H, Dk, window))
        return e;
    if (B == 0) return CSA2_OK;
    if (!score) return fail(CSA2_ERR_INVALID, "csa2_index_score: null pointer");
    const size_t need = index_full_ws_bytes(B, total_len, 1, 0);
    if (!ws || ws_bytes < need || !aligned(ws, 256))
        return fail(CSA2_ERR_WORKSPACE,
                    "csa2_index_score: workspace needs %zu bytes (256-aligned)", need);
    FullWs fw;
    full_ws_layout(B, full_tile_bound(B, total_len), 1, reinterpret_cast<char*>(ws), &fw);
    const unsigned tiles = (unsigned)full_tile_bound(B, total_len);
    return launch_score(H, tiles, reinterpret_cast<hipStream_t>(stream), q, w, keys, row_off, len,
                        B, window, 1, fw, score, max_len);
}

extern "C" int csa2_index_score_block(const signed char* q, const signed char* w,
                                      const signed char* keys, const long long* row_off,
                                      const int* len, int B, int T, int shared, long long max_len,
                                      long long total_len, int H, int Dk, int window, int* score,
                                      void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "csa2_index_score_block";
    if (int e = check_scan_args(fn, q, w, keys, row_off, len, B, max_len, total_len, H, Dk,
                                window))
        return e;
    if (int e = check_block_args(fn, B, T, shared, window)) return e;
    if (B == 0) return CSA2_OK;
    if (!score) return fail(CSA2_ERR_INVALID, "%s: null pointer", fn);
    const size_t need = index_full_block_ws_bytes(B, T, shared, total_len, 0);
    if (!ws || ws_bytes < need || !aligned(ws, 256))
        return fail(CSA2_ERR_WORKSPACE, "%s: workspace needs %zu bytes (256-aligned)", fn, need);
    const int planes = block_planes(T, shared);
    const long long TB = full_tile_bound(B, total_len);
    FullWs fw;
    full_ws_layout(B * planes, planes * TB, 1, reinterpret_cast<char*>(ws), &fw);
    return launch_score_block(H, T, shared, (unsigned)TB, reinterpret_cast<hipStream_t>(stream), q,
                              w, keys, row_off, len, B, window, 1, fw, score, max_len);
}
