/*
 * Plain CPU oracle for the CSA2 sparse-attention decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or constant with the HIP
 * kernels.
 *
 * Every routine is the literal definition written out with plain loops:
 * int64 for the integer index scores, fp64 for attention, exhaustive search
 * for the FP4 rounding.  No blocking, fusion or reordering.
 *
 * Sources (page titles as they appear in the collected pages):
 *  - "DeepSeek V4.1-Flash 552B runs like 16B (CED)", section "Act 2: CSA2 &
 *    Hierarchical Sparse Indexing": one Full pass ranks the context into a
 *    candidate pool, which the later indexing layers rank again.
 *  - "How DeepSeek V4.1 Flash Actually Works", section "The three KV-cache
 *    optimizations", item 2 (Compress Sparse Attention): a layer attends to
 *    512 selected positions and the newest 128 tokens; the pool holds at most
 *    16,384 positions; the KV cache stores 4-bit values.
 *  - "DeepSeek Has Done It Again...", section "Architecture and inference
 *    efficiency": at most 512 history positions next to the newest 128.
 *  - Where the pages leave the arithmetic open, this path fixes it: int8
 *    index keys and queries with exact integer scores,
 *    score = sum_h w_h*max(0, q_h.k), ties broken by lower position, KV stored
 *    as FP4 E2M1 with one E8M0 scale per 32 elements, K = V = latent, softmax
 *    scale 1/sqrt(512), fp32 output.
 *  - The FP4 block-scale rule follows the public OCP Microscaling Formats (MX)
 *    v1.0 specification (shared exponent = floor(log2(amax)) - emax_elem,
 *    emax_elem = 2 for E2M1; elements round to nearest, ties to even,
 *    saturating at the largest magnitude 6).
 *
 * Parity status: every function here is pinned by the CPU tests (brute force,
 * closed forms, published tables); none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* bf16 and FP4 E2M1 / E8M0 (OCP MX v1.0)                                    */
/* ------------------------------------------------------------------------ */

/* A bf16 value is the top 16 bits of an IEEE binary32. */
double oracle_bf16_to_double(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* The eight E2M1 magnitudes, indexed by the low three code bits
 * (OCP MX v1.0, FP4 E2M1: 1 sign, 2 exponent, 1 mantissa bit, bias 1). */
static double e2m1_magnitude(int code3) {
    switch (code3 & 7) {
        case 0: return 0.0;
        case 1: return 0.5;
        case 2: return 1.0;
        case 3: return 1.5;
        case 4: return 2.0;
        case 5: return 3.0;
        case 6: return 4.0;
        default: return 6.0;
    }
}

/* Value of one stored element: (-1)^sign * E2M1[code] * 2^(scale - 127). */
double oracle_fp4_value(int nibble, int scale_byte) {
    double m = e2m1_magnitude(nibble & 7);
    if (nibble & 8) m = -m;
    return ldexp(m, scale_byte - 127);
}

/* Nearest E2M1 magnitude code to y >= 0; on an exact tie the even code wins;
 * anything above 6 saturates to code 7.  Exhaustive search over the grid. */
static int e2m1_round(double y) {
    int best = 0;
    double best_d = fabs(y - e2m1_magnitude(0));
    for (int c = 1; c < 8; ++c) {
        double d = fabs(y - e2m1_magnitude(c));
        if (d < best_d || (d == best_d && (c % 2 == 0))) {
            best = c;
            best_d = d;
        }
    }
    return best;
}

/* Quantise rows of D bf16 values (D a multiple of 32) to FP4 E2M1 codes with
 * one E8M0 scale byte per 32 consecutive elements.
 *   codes : [n_rows][D/2], element 2i in the low nibble of byte i
 *   scales: [n_rows][D/32]
 * Scale rule: X = 2^(floor(log2(amax)) - 2), clamped to the E8M0 range
 * [2^-127, 2^127]; an all-zero block gets the smallest scale byte 0. */
void oracle_fp4_quantize(const uint16_t* x, int64_t n_rows, int D,
                         uint8_t* codes, uint8_t* scales) {
    const int nblk = D / 32;
    for (int64_t r = 0; r < n_rows; ++r) {
        const uint16_t* xr = x + r * (int64_t)D;
        for (int blk = 0; blk < nblk; ++blk) {
            double amax = 0.0;
            for (int i = 0; i < 32; ++i) {
                double v = fabs(oracle_bf16_to_double(xr[blk * 32 + i]));
                if (v > amax) amax = v;
            }
            int shared = -127;
            if (amax > 0.0) {
                int e2;
                (void)frexp(amax, &e2);       /* amax = f * 2^e2, f in [0.5, 1) */
                int floor_log2 = e2 - 1;      /* exact for every finite double */
                shared = floor_log2 - 2;
                if (shared < -127) shared = -127;
                if (shared > 127) shared = 127;
            }
            uint8_t sb = (uint8_t)(shared + 127);
            scales[r * nblk + blk] = sb;
            double X = ldexp(1.0, shared);
            for (int i = 0; i < 32; ++i) {
                uint16_t bits = xr[blk * 32 + i];
                double y = fabs(oracle_bf16_to_double(bits)) / X; /* exact */
                int code = e2m1_round(y);
                if (bits & 0x8000u) code |= 8;  /* sign copied, zeros included */
                int e = blk * 32 + i;
                uint8_t* byte = codes + r * (int64_t)(D / 2) + e / 2;
                if (e % 2 == 0)
                    *byte = (uint8_t)((*byte & 0xF0u) | (uint8_t)code);
                else
                    *byte = (uint8_t)((*byte & 0x0Fu) | (uint8_t)(code << 4));
            }
        }
    }
}

/* Dequantise rows back to fp64 (exact: every value is m * 2^k with m on the
 * E2M1 grid). */
void oracle_fp4_dequantize(const uint8_t* codes, const uint8_t* scales,
                           int64_t n_rows, int D, double* out) {
    const int nblk = D / 32;
    for (int64_t r = 0; r < n_rows; ++r)
        for (int e = 0; e < D; ++e) {
            uint8_t byte = codes[r * (int64_t)(D / 2) + e / 2];
            int nib = (e % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
            out[r * (int64_t)D + e] = oracle_fp4_value(nib, scales[r * nblk + e / 32]);
        }
}

/* ------------------------------------------------------------------------ */
/* Index scores                                                             */
/* ------------------------------------------------------------------------ */

/* s(p) = sum_h w_h * max(0, sum_d q[h][d] * K[p][d]) in int64, for the cache
 * rows listed in `rows` (absolute row numbers of the index-key cache).
 * keys: [*][dk] int8;  q: [H][dk] int8;  w: [H] int8. */
void oracle_index_scores(const int8_t* keys, int dk, const int64_t* rows, int64_t n,
                         const int8_t* q, const int8_t* w, int H, int64_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const int8_t* k = keys + rows[i] * (int64_t)dk;
        int64_t s = 0;
        for (int h = 0; h < H; ++h) {
            int64_t dot = 0;
            for (int d = 0; d < dk; ++d) dot += (int64_t)q[h * dk + d] * (int64_t)k[d];
            if (dot > 0) s += (int64_t)w[h] * dot;
        }
        out[i] = s;
    }
}

/* ------------------------------------------------------------------------ */
/* Order and top-k                                                          */
/* ------------------------------------------------------------------------ */

typedef struct {
    int64_t score;
    int64_t pos;
} scored_pos;

/* p precedes p' iff s(p) > s(p'), or the scores are equal and p < p'. */
static int cmp_rank(const void* a, const void* b) {
    const scored_pos* x = (const scored_pos*)a;
    const scored_pos* y = (const scored_pos*)b;
    if (x->score != y->score) return x->score > y->score ? -1 : 1;
    if (x->pos != y->pos) return x->pos < y->pos ? -1 : 1;
    return 0;
}

static int cmp_pos(const void* a, const void* b) {
    const scored_pos* x = (const scored_pos*)a;
    const scored_pos* y = (const scored_pos*)b;
    if (x->pos != y->pos) return x->pos < y->pos ? -1 : 1;
    return 0;
}

/* The first min(k, n) candidates in rank order, returned in ascending
 * position order with their scores.  Returns the number written. */
int64_t oracle_topk(const int64_t* score, const int64_t* pos, int64_t n, int64_t k,
                    int64_t* out_pos, int64_t* out_score) {
    int64_t keff = k < n ? k : n;
    if (keff <= 0) return 0;
    scored_pos* a = (scored_pos*)malloc((size_t)n * sizeof(scored_pos));
    if (!a) return -1;
    for (int64_t i = 0; i < n; ++i) {
        a[i].score = score[i];
        a[i].pos = pos[i];
    }
    qsort(a, (size_t)n, sizeof(scored_pos), cmp_rank);
    qsort(a, (size_t)keff, sizeof(scored_pos), cmp_pos);
    for (int64_t i = 0; i < keff; ++i) {
        out_pos[i] = a[i].pos;
        out_score[i] = a[i].score;
    }
    free(a);
    return keff;
}

/* ------------------------------------------------------------------------ */
/* Attention over an explicit row set                                       */
/* ------------------------------------------------------------------------ */

/* For each head h over the rows S (K = V = the dequantised latent rows):
 *   t_j = sm_scale * sum_d q[h][d] v[j][d]
 *   out[h][d] = sum_j e^{t_j - m} v[j][d] / sum_j e^{t_j - m},  m = max_j t_j
 *   lse[h] = m + ln sum_j e^{t_j - m}
 * q: [Hq][D] bf16;  v: [S][D] fp64;  out: [Hq][D] fp64;  lse: [Hq].
 * An empty row set gives out = 0 and lse = -inf. */
void oracle_attention(const uint16_t* q, int Hq, int D, const double* v, int64_t S,
                      double sm_scale, double* out, double* lse) {
#pragma omp parallel for schedule(static)
    for (int h = 0; h < Hq; ++h) {
        double* o = out + (int64_t)h * D;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (S == 0) {
            lse[h] = -INFINITY;
            continue;
        }
        double* qh = (double*)malloc((size_t)D * sizeof(double));
        double* t = (double*)malloc((size_t)S * sizeof(double));
        for (int d = 0; d < D; ++d) qh[d] = oracle_bf16_to_double(q[(int64_t)h * D + d]);
        double m = -INFINITY;
        for (int64_t j = 0; j < S; ++j) {
            double acc = 0.0;
            for (int d = 0; d < D; ++d) acc += qh[d] * v[j * D + d];
            t[j] = sm_scale * acc;
            if (t[j] > m) m = t[j];
        }
        double z = 0.0;
        for (int64_t j = 0; j < S; ++j) {
            double e = exp(t[j] - m);
            z += e;
            for (int d = 0; d < D; ++d) o[d] += e * v[j * D + d];
        }
        for (int d = 0; d < D; ++d) o[d] /= z;
        lse[h] = m + log(z);
        free(qh);
        free(t);
    }
}
