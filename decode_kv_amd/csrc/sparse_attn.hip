// csa2_sparse_attn_decode: attention of every query head over the selected
// global positions plus the recent window, reading the FP4 latent cache.
// ("How DeepSeek V4.1 Flash Actually Works", item 2, and "DeepSeek Has Done
// It Again...", "Architecture and inference efficiency": a layer attends to
// 512 positions chosen from the whole history together with the newest 128
// tokens.)  MQA with K = V = the dequantised 512-wide latent row.
//
// Workgroup = (split, sequence, group of 16 heads), four waves, up to four
// 32-row tiles of attended rows.  The launch is one-dimensional so that the
// placement on the eight XCDs (workgroup i on XCD i mod 8) can be chosen: all
// splits of a (sequence, head group) pair, and the combine workgroups of its
// heads, run on one XCD.  All of a workgroup's global loads are issued
// up front (sequence scalars and selection entries, then the raw FP4 rows of
// every tile into registers: 32 bytes of codes and their two scale bytes per
// thread), so the gather latency is paid once.
// Per tile:
//   * every thread dequantises its 64 codes exactly to bf16 and stores them
//     row-major in LDS;
//   * S^T = V q^T on bf16 MFMA (16x16x32), fp32 accumulation, the latent
//     dimension split over the four waves and the partial sums added in LDS;
//   * online softmax in base 2, per head (every wave holds the full scores);
//   * O^T += V^T P^T on bf16 MFMA, each wave owning a quarter of the output
//     dimension, with P split into a bf16 high part and a bf16 residual so the
//     weights carry ~16 significant bits.  The V^T operand comes from the
//     row-major tile through gfx950's transposing LDS read, so the tile is
//     stored once.
// The k-slots of P's MFMA operand are the rows the S^T result left in each
// lane, and V's operand is read with the same row order, so P never moves.
// Computing O^T (M = latent dim, N = head) leaves each lane four consecutive
// outputs of its own head: the softmax rescale needs no lane exchange and the
// partials leave in 16-byte stores.
// Splits write (m, l, O) partials; a second kernel merges them with a
// log-sum-exp combine.
#include <math.h>

#include <mutex>
#include <type_traits>

#include "abi_common.h"
#include "common.h"

namespace csa2 {

constexpr int kAttnThreads = 256;
constexpr int kAttnRows = 32;
constexpr int kAttnD = 512;
constexpr int kHeadsPerWg = 16;
constexpr int kVjdLdMax = kAttnD + 16;  // bf16 per row-major row, at most (1,056 B)
constexpr int kAttnMaxTilesPerWg = 4;   // tiles whose loads one workgroup keeps in flight
constexpr int kAttnMaxRows = 16384;     // k + window
constexpr int kAttnMinWgs = 160;        // workgroups wanted per launch
constexpr int kAttnWideWgs = 256;       // above this many workgroups, the wide layout
constexpr int kAttnMaxSplits = kAttnMaxRows / kAttnRows;   // one tile per split at most

// Eight E2M1 codes (one 32-bit word, element 2i in the low nibble of byte i)
// times 2^d to eight bf16 (element 2i in the low half of word i).  The kernel
// dequantises relative to a per-wave exponent e: d = (scale byte of the block)
// - e.  In general e is the largest scale byte of the rows the wave holds, so
// d <= 0, the values stay between 2^-1 * 2^d and 6, and the power of two is
// applied to the scores and carried with the outputs; when all of the wave's
// scale bytes lie in [2, 200], e = 127 (the absolute scales, d in [-125, 73],
// every value a normal number far from overflow).  v_cvt_scalef32_pk_bf16_fp4 converts the
// two codes of one byte and applies the fp32 scale 2^d, built from its bits
// (subnormal below 2^-126, zero below 2^-149).  Exact whenever d >= -126:
// the results have at most two significant bits.
__device__ __forceinline__ u32x4 fp4x8_to_bf16x8(uint32_t codes, int d) {
    const int eb = d + 127;
    const uint32_t bits = eb > 0 ? (uint32_t)eb << 23 : (eb > -23 ? 0x00400000u >> (-eb) : 0u);
    const float scale = __builtin_bit_cast(float, bits);
    u32x4 r;
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3));
    return r;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// Two layouts of the dequantised tile in LDS.  LDS serves 128 bytes (32
// banks) per cycle; a row is 64 pieces of 16 bytes (8 latent elements).  The
// dequantised stores (eight lanes per cycle, one piece each), the score
// operands (the same piece of rows r..r+7 per eight lanes) and the
// transposing reads (two adjacent pieces of rows 4g..4g+3 per sixteen lanes)
// must each hit eight different bank groups per cycle.
//   * Narrow (few workgroups, latency-bound): thread t dequantises row t >> 3,
//     pieces 8c..8c+7 with c = t & 7, so the loads of a row are contiguous
//     lanes.  Rows are 1,040 bytes apart and piece p sits at position
//     p ^ ((p >> 3) & 7), so thread c writes its j-th piece to position
//     8c + (j ^ c).  The transposing reads meet two-way conflicts.
//   * Wide (more workgroups than CUs, where each instruction counts): lane l
//     of wave w dequantises row 8w + (l & 7), so eight consecutive lanes
//     store to eight rows; rows are 1,056 bytes apart and rows 4..7 mod 8
//     start 16 bytes later.  No conflicts, and every LDS address is a
//     per-lane base plus a constant, with no swizzle arithmetic.
// Both permutations keep pairs of pieces 2i, 2i+1 together, so every read
// stays whole.
template <bool WIDE> constexpr int kVjdLd = WIDE ? kAttnD + 16 : kAttnD + 8;
template <bool WIDE> __device__ __forceinline__ int vjd_row(int r) {
    return WIDE ? r * kVjdLd<WIDE> + 8 * ((r >> 2) & 1) : r * kVjdLd<WIDE>;
}
template <bool WIDE> __device__ __forceinline__ int vjd_piece(int p) {   // offset of piece p
    return WIDE ? 8 * p : 8 * (p ^ ((p >> 3) & 7));
}

// ds_read_b64_tr_b16 at an LDS address (8-byte aligned)
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    return bitcast<u32x2>(__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p)));
}

// Attention of one workgroup over tiles [TPW * split, TPW * split + TPW) of
// its sequence's attended rows.  Every global load the workgroup needs is
// issued before the first tile is processed: the per-sequence scalars and the
// selection entries in one round trip, then the FP4 codes and scales of all
// TPW tiles in a second one, held in registers until their tile's turn.
// The arguments the first round trip needs (the sizes, then the pointers it
// loads from) fill the 64 bytes that arrive in SGPRs with the wave.
// Placement flags of the attention and combine launches.
constexpr int kPlaceSeq = 1;     // sequence b (all head groups and splits) on XCD b mod 8
constexpr int kPlacePlain = 2;   // split partials stored with plain stores (they fit in L2)
// A verify block of T tokens per sequence (flags bits 8 and up hold T, 0
// meaning 1): query row b of the launch is token t = b mod T of sequence b / T, which
// sees the positions before len - (T - 1 - t).  With kBlockShared every token
// of a sequence attends to the sequence's one selection, else row b has its own.
constexpr int kBlockShared = 16;
constexpr int kBlockShift = 8;

// Workgroup i runs on XCD i mod 8.  Pair-major placement puts (sequence, head
// group) pair p on XCD p mod 8: at one sequence its four head groups use four
// XCDs.  Sequence-major placement puts every workgroup of sequence b on XCD
// b mod 8, so that XCD's L2 fetches each FP4 row once for all head groups and
// holds the split partials for the combine.  Returns false past the last pair.
__device__ __forceinline__ bool attn_place(int flags, int B, int HG, int n_splits, int& b,
                                           int& hz, int& split) {
    const int xid = blockIdx.x & 7, xslot = blockIdx.x >> 3;
    const int lp = xslot / n_splits;
    split = xslot - lp * n_splits;
    if (flags & kPlaceSeq) {
        const int bi = lp / HG;
        hz = lp - bi * HG;
        b = bi * 8 + xid;
        return b < B;
    }
    const int pair = lp * 8 + xid;
    b = pair / HG;
    hz = pair - b * HG;
    return pair < B * HG;
}

// BLOCK: a verify block (T > 1 query rows per sequence); the one-token
// instances carry none of its row bookkeeping.
template <int TPW, bool WIDE, bool BLOCK>
__global__ __launch_bounds__(kAttnThreads, 1) void sparse_attn_kernel(
    int B, int Hq, int k, int window, int n_splits, float scale_log2, int flags,
    const long long* __restrict__ row_off, const int* __restrict__ len,
    const int* __restrict__ sel_len, const int* __restrict__ sel_pos,
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv_fp4,
    const uint8_t* __restrict__ kv_scale, float* __restrict__ part_o,
    float* __restrict__ part_ml, float* __restrict__ out, float* __restrict__ lse) {
    // the tile's rows, dequantised, row-major (41 KB of LDS with the
    // partial sums: three workgroups per CU)
    __shared__ __attribute__((aligned(16))) uint16_t s_vjd[kAttnRows * kVjdLdMax];
    constexpr int LD = kVjdLd<WIDE>;
    // S^T partial sums of each wave over its quarter of the latent dimension
    __shared__ f32x4 s_red[kAttnThreads / kWave][2][kWave];
    // per wave: the largest scale byte of the rows it dequantises (all tiles)
    __shared__ int s_e[kAttnThreads / kWave];

    // all splits of one (sequence, head group) pair run on one XCD, where they
    // share the query rows in L2 and the combine of that pair (placed the same
    // way) finds their partials
    const int HG = Hq / kHeadsPerWg;
    int b, hz, split;
    if (!attn_place(flags, B, HG, n_splits, b, hz, split)) return;
    const int tid = threadIdx.x, wave = tid / kWave, l = lane_id();
    const int g = l >> 4, c16 = l & 15;
    const int head = hz * kHeadsPerWg + c16;      // this lane's head
    const int t_begin = split * TPW;

    // round trip 1: sequence scalars, this thread's selection entries, q
    const int bt = BLOCK ? flags >> kBlockShift : 1;
    const int bs = BLOCK ? b / bt : b;                         // the sequence of query row b
    const int bsel = BLOCK && (flags & kBlockShared) ? bs : b;    // the row of its selection
    const int len_b = len[bs] - (BLOCK ? bt - 1 - (b - bs * bt) : 0), sel_b = sel_len[bsel];
    const long long roff = row_off[bs];
    // loads of a tile: thread t takes the 32 bytes of codes of row crow at
    // bytes 32 c8 .. (latent elements 64 c8 ..) and their two scales; each
    // wave takes 8 whole rows
    const int crow = WIDE ? 8 * wave + (l & 7) : tid >> 3, c8 = WIDE ? l >> 3 : tid & 7;
    int spc[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int jc = (t_begin + t) * kAttnRows + crow;
        spc[t] = jc < k ? sel_pos[(size_t)bsel * k + jc] : -1;
    }
    // q . v is split over the latent dimension: wave w owns d in [128w, 128w+128)
    constexpr int kKs = kAttnD / 32 / (kAttnThreads / kWave);   // 4 k-steps per wave
    bf16x8 qb[kKs];
    {
        const uint16_t* qh = q + ((size_t)b * Hq + head) * kAttnD + 32 * kKs * wave + 8 * g;
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks)
            qb[ks] = bitcast<bf16x8>(*reinterpret_cast<const u32x4*>(qh + 32 * ks));
    }
    const int L = max(0, len_b);
    const int win = min(window, L);
    const int nsel = max(0, min(sel_b, k));
    const int S = nsel + win;
    const int ntile = (S + kAttnRows - 1) / kAttnRows;
    const int t_end = min(t_begin + TPW, ntile);
    // p . v is split over the output dimension: wave w owns d-blocks [8w, 8w+8)
    constexpr int kNb = kAttnD / 16 / (kAttnThreads / kWave);   // 8 blocks of 16
    // the results: lane holds head `head`, latent elements 16 (8 wave + nb) + 4 g + (0..3)
    const int d0 = 16 * kNb * wave + 4 * g;
    // oo is in units of 2^(e_fin - 127) (e_fin: the largest scale byte of the
    // workgroup's rows), m_fin and l_fin are the running max and sum of the
    // base-2 scores
    auto emit = [&](const f32x4 (&oo)[kNb], float m_fin, float l_fin, int e_fin) {
        if (n_splits == 1) {
            float* ob = out + ((size_t)b * Hq + head) * kAttnD + d0;
            const float inv = l_fin > 0.f ? 1.f / l_fin : 0.f;
#pragma unroll
            for (int nb = 0; nb < kNb; ++nb) {
                f32x4 r = oo[nb] * inv;
#pragma unroll
                for (int i = 0; i < 4; ++i) r[i] = ldexpf(r[i], e_fin - 127);
                *reinterpret_cast<f32x4*>(ob + 16 * nb) = r;
            }
            if (lse && wave == 0 && g == 0)
                lse[(size_t)b * Hq + head] =
                    l_fin > 0.f ? (m_fin + log2f(l_fin)) * 0.69314718055994531f : -INFINITY;
            return;
        }
        // split partial: unnormalised O, running max and sum.  Only the combine
        // kernel reads them.  When they fit in the XCD's L2 they stay there for
        // it; otherwise they are stored non-temporal (streamed past the caches
        // instead of waiting in L2 for the end-of-kernel write-back).
        const size_t base = ((size_t)b * n_splits + split) * Hq + head;
        float* ob = part_o + base * kAttnD + d0;
        const f32x4 ml = {m_fin, l_fin, (float)e_fin, 0.f};
        if (flags & kPlacePlain) {                           // uniform
#pragma unroll
            for (int nb = 0; nb < kNb; ++nb) *reinterpret_cast<f32x4*>(ob + 16 * nb) = oo[nb];
            if (wave == 0 && g == 0) *reinterpret_cast<f32x4*>(part_ml + base * 4) = ml;
        } else {
#pragma unroll
            for (int nb = 0; nb < kNb; ++nb)
                __builtin_nontemporal_store(oo[nb], reinterpret_cast<f32x4*>(ob + 16 * nb));
            if (wave == 0 && g == 0)
                __builtin_nontemporal_store(ml, reinterpret_cast<f32x4*>(part_ml + base * 4));
        }
    };
    if (t_begin >= t_end) {                              // uniform: a split past the attended rows
        f32x4 z[kNb];
#pragma unroll
        for (int nb = 0; nb < kNb; ++nb) z[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        emit(z, -INFINITY, 0.f, 0);
        return;
    }

    // round trip 2: the raw rows of every tile, in 16-byte loads (a row of an
    // invalid position reads row 0 and is staged as zeros)
    auto pos_of = [&](int j, int p) -> long long {
        if (j < nsel) return p;
        if (j < S) return (long long)(L - win + (j - nsel));
        return -1;
    };
    u32x4 rc0[TPW], rc1[TPW];
    uint32_t rsb[TPW];                                   // scale bytes of elements 0..31, 32..63
    uint32_t cok = 0;                                    // per tile: row valid
    long long rrow[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {                      // the scale bytes first: the wave's
        const long long pc = pos_of((t_begin + t) * kAttnRows + crow, spc[t]);   // exponent
        cok |= (uint32_t)(pc >= 0) << t;                 // needs them before any tile
        rrow[t] = roff + (pc >= 0 ? pc : 0);
        rsb[t] = *reinterpret_cast<const uint16_t*>(kv_scale + rrow[t] * (kAttnD / 32) + 2 * c8);
    }
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const uint8_t* cp = kv_fp4 + rrow[t] * (kAttnD / 2) + 32 * c8;
        rc0[t] = *reinterpret_cast<const u32x4*>(cp);
        rc1[t] = *reinterpret_cast<const u32x4*>(cp + 16);
    }
    // the wave's exponent: the largest scale byte of its valid rows in all of
    // the workgroup's tiles (a wave holds the same 8 rows of every tile), or
    // 127 when every such byte lies in [2, 200]: the absolute scales are then
    // exact and overflow-free (values within [2^-126, 6 * 2^73], every
    // product and sum far inside fp32) and no cross-lane maximum is needed
    int ew = 0;
    bool outside = false;
#pragma unroll
    for (int t = 0; t < TPW; ++t)
        if ((cok >> t) & 1u) {
            const int b0 = (int)(rsb[t] & 0xFFu), b1 = (int)(rsb[t] >> 8);
            ew = max(ew, max(b0, b1));
            outside |= min(b0, b1) < 2 || max(b0, b1) > 200;
        }
    if (__ballot(outside) == 0)                          // uniform
        ew = 127;
    else
        ew = __builtin_amdgcn_readfirstlane((int)wave_max((float)ew));
    if (l == 0) s_e[wave] = ew;

    f32x4 o[kNb];                                        // set by the first tile's P.V
    float m_run = -INFINITY, l_run = 0.f;
    int ea = 0, eb = 0, etop = 0;                        // exponents, read after the first barrier

#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int tile = t_begin + t;
        if (t > 0 && tile >= t_end) break;                  // uniform; tile t_begin exists
        if (t > 0) __syncthreads();                          // previous tile's LDS reads are done
        {
            // dequantise this thread's 64 elements of row crow straight from
            // the loaded registers (an invalid row is zeros, scale byte 0)
            const u32x4 z = {0u, 0u, 0u, 0u};
            const bool ok = (cok >> t) & 1u;
            const u32x4 a = ok ? rc0[t] : z, bq = ok ? rc1[t] : z;
            const int sbp = ok ? (int)rsb[t] : 0;
            // pieces 8 c8 + j and 8 c8 + 4 + j (narrow: positions 8 c8 + (j ^ c8) ..)
            uint16_t* vr = s_vjd + vjd_row<WIDE>(crow) + 64 * c8;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int p0 = WIDE ? 8 * j : 8 * (j ^ c8);
                const int p1 = WIDE ? 32 + 8 * j : 8 * ((4 + j) ^ c8);
                *reinterpret_cast<u32x4*>(vr + p0) = fp4x8_to_bf16x8(a[j], (sbp & 0xFF) - ew);
                *reinterpret_cast<u32x4*>(vr + p1) = fp4x8_to_bf16x8(bq[j], (sbp >> 8) - ew);
            }
        }
        __syncthreads();

        // partial S^T[row][head] over this wave's quarter of the latent dimension
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        {
            // rows c16 and 16 + c16 (the same offset of 16 rows further on)
            // latent elements 128 wave + 32 ks + 8 g .. (piece 16 wave + 4 ks + g)
            const uint16_t* r0 = s_vjd + vjd_row<WIDE>(c16) + (WIDE ? 32 * kKs * wave + 8 * g : 0);
            const uint16_t* r1 = r0 + 16 * LD;
#pragma unroll
            for (int ks = 0; ks < kKs; ++ks) {
                const int pc = WIDE ? 32 * ks : vjd_piece<WIDE>(4 * kKs * wave + 4 * ks + g);
                const bf16x8 a0 = bitcast<bf16x8>(*reinterpret_cast<const u32x4*>(r0 + pc));
                const bf16x8 a1 = bitcast<bf16x8>(*reinterpret_cast<const u32x4*>(r1 + pc));
                s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qb[ks], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qb[ks], s1, 0, 0, 0);
            }
        }
        s_red[wave][0][l] = s0;
        s_red[wave][1][l] = s1;
        __syncthreads();
        // this wave's V^T operands of the P.V product (latent elements d0 + c16
        // of rows 4g..4g+3 and 16+4g..16+4g+3, d0 = 16 (8 wave + nb)), read
        // before the softmax so their LDS latency overlaps it.  The gfx950
        // transposing LDS read works in groups of 16 lanes: lane 4a + c of a
        // group receives, as element e, the 16-bit value at offset c of the
        // 8 bytes addressed by lane a + 4e of the group.  So lane (g, 4a' + c')
        // addresses row 4g + a' at elements d0 + 4c' .. d0 + 4c' + 3.
        bf16x8 bv[kNb];
        {
            // latent elements d0 + 4 (c16 & 3) ..: half c16 & 1 of piece d0 / 8 + (c16 & 3) / 2
            const uint16_t* vt = s_vjd + vjd_row<WIDE>(4 * g + (c16 >> 2)) +
                                 (WIDE ? 16 * kNb * wave + 4 * (c16 & 3) : 4 * (c16 & 1));
#pragma unroll
            for (int nb = 0; nb < kNb; ++nb) {
                const int pc = WIDE ? 16 * nb : vjd_piece<WIDE>(2 * kNb * wave + 2 * nb + ((c16 & 3) >> 1));
                const u32x2 lo = lds_read_tr16(vt + pc);
                const u32x2 hi = lds_read_tr16(vt + 16 * LD + pc);
                bv[nb] = bitcast<bf16x8>(u32x4{lo[0], lo[1], hi[0], hi[1]});
            }
        }
        s0 = s_red[0][0][l] + s_red[1][0][l] + s_red[2][0][l] + s_red[3][0][l];
        s1 = s_red[0][1][l] + s_red[1][1][l] + s_red[2][1][l] + s_red[3][1][l];
        if (t == 0) {
            // rows 4g..4g+3 were dequantised by wave g >> 1, rows 16+4g.. by
            // wave 2 + (g >> 1); etop is the workgroup's largest exponent
            ea = s_e[g >> 1];
            eb = s_e[2 + (g >> 1)];
            etop = max(max(s_e[0], s_e[1]), max(s_e[2], s_e[3]));
        }

        // every wave now holds the full scores: head c16, rows 4g+i and 16+4g+i
        // (the scores of the relative values times their wave's 2^(e - 127))
        const int jt = tile * kAttnRows;
        float ts[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ts[i] = ldexpf(s0[i] * scale_log2, ea - 127);
            ts[4 + i] = ldexpf(s1[i] * scale_log2, eb - 127);
        }
        if (jt + kAttnRows > S) {                        // uniform: rows past S weigh 0
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (jt + 4 * g + i >= S) ts[i] = -INFINITY;
                if (jt + 16 + 4 * g + i >= S) ts[4 + i] = -INFINITY;
            }
        }
        float tmax = ts[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, ts[i]);
        tmax = rows4_max(tmax);
        const float m_new = fmaxf(m_run, tmax);   // finite: every tile has a valid row
        float p[8], psum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[i] = __builtin_amdgcn_exp2f(ts[i] - m_new);   // <= 0; -inf gives 0
            psum += p[i];
        }
        psum = rows4_sum(psum);
        if (t == 0) {                              // nothing accumulated yet
            l_run = psum;
        } else {
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run = l_run * alpha + psum;
#pragma unroll
            for (int nb = 0; nb < kNb; ++nb) o[nb] *= alpha;   // this lane's head
        }
        m_run = m_new;

        u32x4 ph_u, pl_u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // two weights per conversion: the bf16 high parts, then the bf16
            // residuals (each residual is exact in fp32 before rounding).  A
            // row's weight times 2^(its wave's exponent - etop) puts every row's
            // relative values on the workgroup's common scale 2^(etop - 127).
            const int sh = (i < 2 ? ea : eb) - etop;
            const f32x2 pp = {ldexpf(p[2 * i], sh), ldexpf(p[2 * i + 1], sh)};
            const uint32_t hu = bitcast<uint32_t>(__builtin_convertvector(pp, bf16x2));
            const f32x2 hf = {__uint_as_float(hu << 16), __uint_as_float(hu & 0xFFFF0000u)};
            ph_u[i] = hu;
            pl_u[i] = bitcast<uint32_t>(__builtin_convertvector(pp - hf, bf16x2));
        }
        const bf16x8 ph = bitcast<bf16x8>(ph_u), pl = bitcast<bf16x8>(pl_u);
#pragma unroll
        for (int nb = 0; nb < kNb; ++nb) {
            // O^T[d][head]: A = V^T (M = latent dim), B = P^T (N = head)
            const f32x4 acc = t == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : o[nb];
            o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bv[nb], ph, acc, 0, 0, 0);
            o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bv[nb], pl, o[nb], 0, 0, 0);
        }
    }

    emit(o, m_run, l_run, etop);
}

// Log-sum-exp merge of the split partials: one workgroup per (head, sequence),
// on the XCD of that head's attention workgroups (workgroup i runs on XCD
// i mod 8), 128 threads x 4 output elements.  Each thread issues the loads of its
// partial outputs of CH splits (indices past the last split reread it and get
// weight 0) and, for split s = thread, that split's (m, l, e), all before any of
// them is used, so the merge costs one memory round trip; splits beyond CH
// follow in further chunks.  CH is the smallest of 8, 16, 24, 32 that covers
// the splits when it can.
// The running maxima and sums are reduced once per workgroup: the split
// weights 2^(m_s - M) go to LDS and every thread reads them four at a time.
// An empty split has m = -inf and weight 0.  The pointers are not
// __restrict__ so that the loads keep their order around the empty asm.
template <int CH>
__global__ __launch_bounds__(128) void attn_combine_kernel(const float* part_o,
                                                           const float* part_ml,
                                                           int Hq, int n_splits,
                                                           float* __restrict__ out,
                                                           float* __restrict__ lse, int B,
                                                           int flags) {
    __shared__ __attribute__((aligned(16))) float s_w[kAttnMaxSplits + 32];   // zero-padded to CH
    __shared__ float s_red[3][2];
    // the combine of head h of a pair runs on the pair's XCD (attn_place with
    // one "split" per head of the pair)
    const int HG = Hq / kHeadsPerWg;
    int b, hz, hl;
    if (!attn_place(flags, B, HG, kHeadsPerWg, b, hz, hl)) return;
    const int h = hz * kHeadsPerWg + hl, tid = threadIdx.x;
    const size_t row0 = (size_t)b * n_splits * Hq + h;          // split s at row0 + s * Hq
    f32x4 os[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
        const int s = min(u, n_splits - 1);
        os[u] = *reinterpret_cast<const f32x4*>(part_o + (row0 + (size_t)s * Hq) * kAttnD + 4 * tid);
    }
    const f32x4 ml = *reinterpret_cast<const f32x4*>(
        part_ml + (row0 + (size_t)min(tid, n_splits - 1) * Hq) * 4);   // used for tid < n_splits
    asm volatile("" ::: "memory");
    // A split's partial is (m_s, l_s, e_s) and O_s in units of 2^(e_s - 127).
    // M = max m_s and Ex = max e_s over the splits; w_s = 2^(m_s - M) (0 for an
    // empty split); lsum = sum w_s l_s; split s enters the output sum with
    // w_s 2^(e_s - Ex) (kept in LDS, zero-padded to a multiple of CH) and the
    // sum is scaled by 2^(Ex - 127) at the end
    const int n_pad = (n_splits + CH - 1) / CH * CH;
    float M, lsum;
    int Ex;
    if (n_pad <= kWave) {                                       // uniform: wave 0 alone
        if (tid < kWave) {
            const bool in = tid < n_splits;
            const float m = in ? ml.x : -INFINITY;
            const float Mw = wave_max(m);
            const float Ew = wave_max(in ? ml.z : 0.f);
            const float w = (in && Mw != -INFINITY) ? exp2f(m - Mw) : 0.f;
            const float ls = wave_sum(w * (in ? ml.y : 0.f));
            s_w[tid] = in ? ldexpf(w, (int)(ml.z - Ew)) : 0.f;
            if (tid == 0) {
                s_red[0][0] = Mw;
                s_red[1][0] = ls;
                s_red[2][0] = Ew;
            }
        }
        __syncthreads();
        M = s_red[0][0];
        lsum = s_red[1][0];
        Ex = (int)s_red[2][0];
    } else {
        float mloc = tid < n_splits ? ml.x : -INFINITY;
        float eloc = tid < n_splits ? ml.z : 0.f;
        for (int s = tid + 128; s < n_splits; s += 128) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(part_ml + (row0 + (size_t)s * Hq) * 4);
            mloc = fmaxf(mloc, v.x);
            eloc = fmaxf(eloc, v.z);
        }
        mloc = wave_max(mloc);
        eloc = wave_max(eloc);
        if ((tid & (kWave - 1)) == 0) {
            s_red[0][tid / kWave] = mloc;
            s_red[2][tid / kWave] = eloc;
        }
        __syncthreads();
        M = fmaxf(s_red[0][0], s_red[0][1]);
        Ex = (int)fmaxf(s_red[2][0], s_red[2][1]);
        float lpart = 0.f;
        for (int s = tid; s < n_pad; s += 128) {
            float w = 0.f;
            if (s < n_splits && M != -INFINITY) {
                f32x4 v = ml;
                if (s >= 128) v = *reinterpret_cast<const f32x4*>(part_ml + (row0 + (size_t)s * Hq) * 4);
                const float ws = exp2f(v.x - M);
                lpart += ws * v.y;
                w = ldexpf(ws, (int)v.z - Ex);
            }
            s_w[s] = w;
        }
        lpart = wave_sum(lpart);
        if ((tid & (kWave - 1)) == 0) s_red[1][tid / kWave] = lpart;
        __syncthreads();
        lsum = s_red[1][0] + s_red[1][1];
    }
    float* o = out + ((size_t)b * Hq + h) * kAttnD + 4 * tid;
    if (M == -INFINITY) {                                       // nothing attended
        *reinterpret_cast<f32x4*>(o) = f32x4{0.f, 0.f, 0.f, 0.f};
        if (lse && tid == 0) lse[(size_t)b * Hq + h] = -INFINITY;
        return;
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < n_splits; c0 += CH) {
        if (c0 > 0) {
#pragma unroll
            for (int u = 0; u < CH; ++u) {
                const int s = min(c0 + u, n_splits - 1);
                os[u] = *reinterpret_cast<const f32x4*>(part_o + (row0 + (size_t)s * Hq) * kAttnD + 4 * tid);
            }
        }
#pragma unroll
        for (int u4 = 0; u4 < CH; u4 += 4) {
            const f32x4 w = *reinterpret_cast<const f32x4*>(s_w + c0 + u4);   // zero past n_splits
#pragma unroll
            for (int i = 0; i < 4; ++i) acc += w[i] * os[u4 + i];
        }
    }
    f32x4 r = acc / lsum;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = ldexpf(r[i], Ex - 127);
    *reinterpret_cast<f32x4*>(o) = r;
    if (lse && tid == 0) lse[(size_t)b * Hq + h] = (M + log2f(lsum)) * 0.69314718055994531f;
}

// Tiles per workgroup: the most (up to 4) that still leave at least
// kAttnMinWgs workgroups for the chip, so small batches spread the selection
// over many CUs and large batches amortise each workgroup's set-up.
int sparse_attn_tiles_per_wg(int B, int Hq, int k, int window) {
    const int tiles = (k + window + kAttnRows - 1) / kAttnRows;
    const long long wgs = (long long)(B > 0 ? B : 1) * ((Hq + kHeadsPerWg - 1) / kHeadsPerWg);
    for (int tpw = kAttnMaxTilesPerWg; tpw > 1; tpw /= 2)
        if (wgs * ((tiles + tpw - 1) / tpw) >= kAttnMinWgs) return tpw;
    return 1;
}

int sparse_attn_splits(int B, int Hq, int k, int window) {
    const int tiles = (k + window + kAttnRows - 1) / kAttnRows;
    const int tpw = sparse_attn_tiles_per_wg(B, Hq, k, window);
    const int ns = (tiles + tpw - 1) / tpw;
    return ns < 1 ? 1 : ns;
}

// Workspace: the partial O, then (m, l, e, -), of every (sequence, split, head).
static size_t attn_ws_layout(int B, int Hq, int ns, char* base, float** part_o,
                             float** part_ml) {
    const size_t n = (size_t)B * ns * Hq;
    const size_t o_bytes = round_up(n * kAttnD * 4, 256);
    if (base) {
        *part_o = reinterpret_cast<float*>(base);
        *part_ml = reinterpret_cast<float*>(base + o_bytes);
    }
    return o_bytes + round_up(n * 4 * 4, 256);
}

size_t sparse_attn_ws_bytes(int B, int Hq, int D, int k, int window) {
    (void)D;
    const int ns = sparse_attn_splits(B, Hq, k, window);
    if (ns <= 1) return 0;
    return attn_ws_layout(B, Hq, ns, nullptr, nullptr, nullptr);
}

// The entry points' shared body: argument checks, then the attention and
// combine launches with the split partials in the scratch that get_ws(need,
// &ptr) supplies once the sizes are known to be valid.  fn names the entry
// point in error messages.
// T and shared describe a verify block (T == 1: one token per sequence); the
// launch then has B * T query rows.
template <typename GetWs>
static int attn_decode(const char* fn, const void* q_bf16, const unsigned char* kv_fp4,
                       const unsigned char* kv_scale, const long long* row_off, const int* len,
                       long long max_len, const int* sel_pos, const int* sel_len, int B, int T,
                       int shared, int Hq, int D, int k, int window, float sm_scale, float* out,
                       float* lse, GetWs get_ws, void* stream) {
    if (B < 0 || max_len < 0 || k < 0 || window < 0)
        return fail(CSA2_ERR_INVALID, "%s: negative size", fn);
    if (T < 1 || shared < 0 || shared > 1)
        return fail(CSA2_ERR_INVALID, "%s: T < 1 or shared not 0/1", fn);
    if (T > 1024) return fail(CSA2_ERR_UNSUPPORTED, "%s: T > 1024", fn);
    if (B == 0) return CSA2_OK;
    if ((long long)B * T > 65535) return fail(CSA2_ERR_UNSUPPORTED, "%s: B * T > 65535", fn);
    B *= T;                                              // query rows of the launch
    if (!q_bf16 || !kv_fp4 || !kv_scale || !row_off || !len || !sel_len || !out ||
        (k > 0 && !sel_pos))
        return fail(CSA2_ERR_INVALID, "%s: null pointer", fn);
    if (D != kAttnD) return fail(CSA2_ERR_UNSUPPORTED, "%s: D must be 512", fn);
    if (Hq < 16 || Hq % 16 != 0)
        return fail(CSA2_ERR_INVALID, "%s: Hq must be a positive multiple of 16", fn);
    if (B > 65535 || Hq > 1024) return fail(CSA2_ERR_UNSUPPORTED, "%s: B or Hq too large", fn);
    // the kernel reads a row's codes in 16-byte pieces and its scale bytes in
    // pairs, and stores the outputs in 16-byte pieces
    if (!aligned(q_bf16, 16) || !aligned(kv_fp4, 16) || !aligned(kv_scale, 2) ||
        !aligned(out, 16) || !aligned(row_off, 8) || !aligned(len, 4) || !aligned(sel_len, 4) ||
        !aligned(sel_pos, 4) || !aligned(lse, 4))
        return fail(CSA2_ERR_INVALID, "%s: misaligned pointer", fn);
    if ((long long)k + window > kAttnMaxRows)
        return fail(CSA2_ERR_UNSUPPORTED, "%s: k + window > %d", fn, kAttnMaxRows);
    const int tpw = sparse_attn_tiles_per_wg(B, Hq, k, window);
    const int ns = sparse_attn_splits(B, Hq, k, window);
    void* ws = nullptr;
    if (int e = get_ws(sparse_attn_ws_bytes(B, Hq, D, k, window), &ws)) return e;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    float* part_o = nullptr;
    float* part_ml = nullptr;
    if (ns > 1) attn_ws_layout(B, Hq, ns, reinterpret_cast<char*>(ws), &part_o, &part_ml);
    const float scale_log2 = sm_scale * 1.4426950408889634f;
    const int HG = Hq / kHeadsPerWg, npairs = B * HG;
    // sequence-major placement from 8 sequences on; plain partial stores when
    // one XCD's share of the partials fits in 3 of its 4 MB of L2
    const bool seq = B >= 8;
    const long long per_xcd = seq ? (long long)((B + 7) / 8) * HG : (npairs + 7) / 8;
    const bool plain = per_xcd * ns * kHeadsPerWg * (kAttnD * 4 + 16) <= (3ll << 20);
    const int flags = (seq ? kPlaceSeq : 0) | (plain ? kPlacePlain : 0) |
                      (T > 1 && shared ? kBlockShared : 0) | (T > 1 ? T << kBlockShift : 0);
    const int pr = seq ? (int)((B + 7) / 8) * HG : (npairs + 7) / 8;   // slots per XCD / splits
    const dim3 grid(8 * pr * ns), blk(kAttnThreads);
    const uint16_t* q16 = reinterpret_cast<const uint16_t*>(q_bf16);
    auto launch = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, grid, blk, 0, s, B, Hq, k, window, ns, scale_log2, flags,
                           row_off, len, sel_len, sel_pos, q16, kv_fp4, kv_scale, part_o, part_ml,
                           out, lse);
    };
    const bool wide = (long long)npairs * ns > kAttnWideWgs;
    auto launch_tpw = [&](auto blk) {
        constexpr bool BLK = decltype(blk)::value;
        switch (tpw) {
            case 1: wide ? launch(sparse_attn_kernel<1, true, BLK>) : launch(sparse_attn_kernel<1, false, BLK>); break;
            case 2: wide ? launch(sparse_attn_kernel<2, true, BLK>) : launch(sparse_attn_kernel<2, false, BLK>); break;
            default: wide ? launch(sparse_attn_kernel<4, true, BLK>) : launch(sparse_attn_kernel<4, false, BLK>); break;
        }
    };
    if (T > 1)
        launch_tpw(std::true_type{});
    else
        launch_tpw(std::false_type{});
    if (int e = launch_status(fn)) return e;
    if (ns > 1) {
        const dim3 cg(8 * pr * kHeadsPerWg), cb(128);
        if (ns <= 8)
            hipLaunchKernelGGL(attn_combine_kernel<8>, cg, cb, 0, s, part_o, part_ml, Hq, ns, out, lse, B, flags);
        else if (ns <= 16)
            hipLaunchKernelGGL(attn_combine_kernel<16>, cg, cb, 0, s, part_o, part_ml, Hq, ns, out, lse, B, flags);
        else if (ns <= 24)
            hipLaunchKernelGGL(attn_combine_kernel<24>, cg, cb, 0, s, part_o, part_ml, Hq, ns, out, lse, B, flags);
        else
            hipLaunchKernelGGL(attn_combine_kernel<32>, cg, cb, 0, s, part_o, part_ml, Hq, ns, out, lse, B, flags);
        return launch_status(fn);
    }
    return CSA2_OK;
}

// ---- the allocation-free variant ------------------------------------------------
// The split partials live in a file-scope device array of kAttnStaticScratch
// bytes.  In host code the array's name is only a stand-in: its device
// address is looked up once per device, with that device current, and that
// address is what the kernels receive.
constexpr size_t kAttnStaticScratch = CSA2_ATTN_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

}  // namespace csa2

static __device__ __align__(256) unsigned char scratch[csa2::kAttnStaticScratch];

namespace csa2 {

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (the device `stream`
// runs on must be the current one).
static int static_scratch(const char* fn, hipStream_t stream, void** out) {
    int dev = 0;
    if (int e = hip_status(hipGetDevice(&dev), "hipGetDevice")) return e;
    if (stream) {
        hipDevice_t sdev = 0;
        if (int e = hip_status(hipStreamGetDevice(stream, &sdev), "hipStreamGetDevice")) return e;
        if ((int)sdev != dev)
            return fail(CSA2_ERR_INVALID,
                        "%s: the stream belongs to device %d, not to the current device %d", fn,
                        (int)sdev, dev);
    }
    if (dev < 0 || dev >= kMaxDevices)
        return fail(CSA2_ERR_UNSUPPORTED, "%s: device id %d >= %d", fn, dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (int e = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)),
                               "hipGetSymbolAddress(scratch)"))
            return e;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return CSA2_OK;
}

}  // namespace csa2

using namespace csa2;

extern "C" int csa2_sparse_attn_decode(const void* q_bf16, const unsigned char* kv_fp4,
                                       const unsigned char* kv_scale, const long long* row_off,
                                       const int* len, long long max_len, const int* sel_pos,
                                       const int* sel_len, int B, int Hq, int D, int k,
                                       int window, float sm_scale, float* out, float* lse,
                                       void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "csa2_sparse_attn_decode";
    auto caller_ws = [&](size_t need, void** p) -> int {
        if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 256)))
            return fail(CSA2_ERR_WORKSPACE, "%s: workspace needs %zu bytes (256-aligned)", fn,
                        need);
        *p = ws;
        return CSA2_OK;
    };
    return attn_decode(fn, q_bf16, kv_fp4, kv_scale, row_off, len, max_len, sel_pos, sel_len, B,
                       1, 0, Hq, D, k, window, sm_scale, out, lse, caller_ws, stream);
}

extern "C" int csa2_sparse_attn_decode_static(const void* q_bf16, const unsigned char* kv_fp4,
                                              const unsigned char* kv_scale,
                                              const long long* row_off, const int* len,
                                              long long max_len, const int* sel_pos,
                                              const int* sel_len, int B, int Hq, int D, int k,
                                              int window, float sm_scale, float* out, float* lse,
                                              void* stream) {
    const char* fn = "csa2_sparse_attn_decode_static";
    auto static_ws = [&](size_t need, void** p) -> int {
        if (need > kAttnStaticScratch)
            return fail(CSA2_ERR_UNSUPPORTED,
                        "%s: these sizes need %zu bytes of scratch; the static scratch holds %zu",
                        fn, need, kAttnStaticScratch);
        if (need == 0) {
            *p = nullptr;
            return CSA2_OK;
        }
        return static_scratch(fn, reinterpret_cast<hipStream_t>(stream), p);
    };
    return attn_decode(fn, q_bf16, kv_fp4, kv_scale, row_off, len, max_len, sel_pos, sel_len, B,
                       1, 0, Hq, D, k, window, sm_scale, out, lse, static_ws, stream);
}

extern "C" int csa2_sparse_attn_decode_block(const void* q_bf16, const unsigned char* kv_fp4,
                                             const unsigned char* kv_scale,
                                             const long long* row_off, const int* len,
                                             long long max_len, const int* sel_pos,
                                             const int* sel_len, int B, int T, int shared, int Hq,
                                             int D, int k, int window, float sm_scale, float* out,
                                             float* lse, void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "csa2_sparse_attn_decode_block";
    auto caller_ws = [&](size_t need, void** p) -> int {
        if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 256)))
            return fail(CSA2_ERR_WORKSPACE, "%s: workspace needs %zu bytes (256-aligned)", fn,
                        need);
        *p = ws;
        return CSA2_OK;
    };
    return attn_decode(fn, q_bf16, kv_fp4, kv_scale, row_off, len, max_len, sel_pos, sel_len, B,
                       T, shared, Hq, D, k, window, sm_scale, out, lse, caller_ws, stream);
}
