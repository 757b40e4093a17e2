/*
 * csa2.h -- C ABI of libcsa2.so: the decode hot path of CSA2 hierarchical
 * sparse attention on AMD MI355X (gfx950).
 *
 * What the path computes (page title, section):
 *  - "DeepSeek V4.1-Flash 552B runs like 16B (CED)", "Act 2: CSA2 &
 *    Hierarchical Sparse Indexing": a Full indexing layer searches the whole
 *    context and builds a candidate pool; later layers search only the pool
 *    (Reindex) or reuse what is already known (Reuse).
 *  - "How DeepSeek V4.1 Flash Actually Works", "The three KV-cache
 *    optimizations", item 2: attention reads the 512 most relevant KV entries
 *    plus a local 128-token window; one indexing layer yields up to 16,384
 *    candidate positions; KV values are stored in FP4.
 *  - "DeepSeek Has Done It Again...", "Architecture and inference efficiency":
 *    up to 512 global positions alongside the 128 most recent tokens.
 * Readings this library fixes where the pages are silent: int8 index keys
 * (one 64-byte key per token, shared by all index heads) and int8 queries;
 * score(p) = sum_h w_h * max(0, q_h . K[p]) exact in int32; rank order =
 * score descending, then position ascending; FP4 E2M1 codes with one E8M0
 * scale byte per 32 consecutive elements (OCP MX v1.0); attention is MQA with
 * K = V = the dequantised latent row.
 *
 * Conventions shared by every entry point
 *  - All array pointers are DEVICE pointers owned by the caller.  The library
 *    allocates no device memory and keeps no state between calls; scratch
 *    memory is a caller workspace of csa2_workspace_bytes() bytes.
 *  - Every call is asynchronous on `stream` (a hipStream_t passed as void*,
 *    NULL = the default stream) and returns after enqueueing its kernels.
 *  - Arguments are validated on the host before anything is launched; on an
 *    error nothing is launched and a negative status is returned, with a
 *    message available from csa2_last_error() (thread-local).
 *  - B sequences share one index-key cache and one KV cache per layer.
 *    Sequence b owns cache rows row_off[b] .. row_off[b] + len[b] - 1 (row =
 *    token position + row_off[b]).  row_off and len live in device memory so
 *    that lengths can advance without host involvement; max_len and total_len
 *    are host-side upper bounds (max_b len[b] and sum_b len[b]) used only for
 *    grid and workspace sizing.  A length above its bound is undefined
 *    behaviour.
 *  - Window: positions [L - window, L) are the local window.  Only positions
 *    [0, E) with E = max(0, L - window) are eligible for the pool and the
 *    selection, so a position is never attended twice.
 *  - Position lists (pool, selection) are ascending; entries past the valid
 *    count are filled with -1.
 *  - Integer outputs are deterministic and independent of the launch shape.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum csa2_status {
    CSA2_OK = 0,
    CSA2_ERR_INVALID = -1,     /* bad pointer, size or alignment            */
    CSA2_ERR_WORKSPACE = -2,   /* workspace missing or too small            */
    CSA2_ERR_UNSUPPORTED = -3, /* valid but not implemented (e.g. D != 512) */
    CSA2_ERR_HIP = -4          /* HIP runtime or launch error               */
};

/* Operation codes for csa2_workspace_bytes(). */
enum csa2_op {
    CSA2_OP_INDEX_FULL = 1,
    CSA2_OP_SELECT_TOPK = 2,
    CSA2_OP_SPARSE_ATTN = 3
};

/* Text of the last non-OK status on the calling thread ("" if none). */
const char* csa2_last_error(void);

/* Library version string. */
const char* csa2_version(void);

/* Bytes of device workspace `op` needs for the given sizes (0 if none).
 * Arguments an op does not use are ignored.  Returns 0 and sets the last
 * error on invalid sizes. */
size_t csa2_workspace_bytes(int op, int B, long long max_len, long long total_len,
                            int H, int P, int k, int Hq, int D, int window);

/*
 * csa2_kv_append_fp4 -- quantise n bf16 latent rows into the FP4 cache.
 * ("DeepSeek V4.1-Flash 552B runs like 16B (CED)", "Act 3": FP4 main KV
 * caching; "How DeepSeek V4.1 Flash Actually Works", item 2: KV compressed
 * from FP8 to FP4.)
 *   x_bf16   [n][D] bf16, row-major, 16-byte aligned.
 *   dst_row  [n] int64: destination row of each input row (any row of the
 *            arrays below; rows must be distinct within one call).
 *   kv_fp4   [rows][D/2] uint8: element 2i in the low nibble of byte i.
 *   kv_scale [rows][D/32] uint8: E8M0 scale of each block of 32 elements.
 * Per block: X = 2^(floor(log2 amax) - 2) clamped to [2^-127, 2^127] (E8M0
 * byte 0 for an all-zero or subnormal block); each element is |x|/X rounded
 * to the nearest E2M1 magnitude {0,.5,1,1.5,2,3,4,6}, ties to the even code,
 * saturating at 6; the sign bit is copied (also for zero).  Exact integer
 * arithmetic on the bf16 bits, so the bytes are bit-reproducible.
 * Errors: INVALID for null pointers, n < 0, D % 32 != 0 or misaligned x.
 * n == 0 is a no-op.
 */
int csa2_kv_append_fp4(const void* x_bf16, const long long* dst_row, int n, int D,
                       unsigned char* kv_fp4, unsigned char* kv_scale, void* stream);

/*
 * csa2_index_full -- Full mode: score every eligible position of each
 * sequence and keep the first P_eff = min(P, E_b) positions under the rank
 * order as the candidate pool.
 * ("DeepSeek V4.1-Flash 552B runs like 16B (CED)", "Act 2": the first
 * full-mode indexing layer searches the large context and builds a candidate
 * pool; "How DeepSeek V4.1 Flash Actually Works", item 2: up to 16,384
 * candidate positions.)
 *   q        [B][H][Dk] int8 index queries (one per sequence), 16-byte aligned.
 *   w        [B][H] int8 per-head weights in [0, 15].
 *   keys     index-key cache, row r at keys + r*Dk (int8), 16-byte aligned.
 *   row_off  [B] int64, len [B] int32 (device).
 *   pool_pos [B][P] int32 out: pool positions, ascending, tail -1.
 *   pool_score [B][P] int32 out: score of each pool entry, tail -1.
 *   pool_len [B] int32 out: P_eff.
 *   k        0, or the size of the Full layer's own selection (1 <= k <= P).
 *   sel_pos  [B][k] int32 out when k > 0 (else ignored, may be NULL): the
 *            first min(k, P_eff) positions under the same rank order,
 *            ascending, tail -1 -- exactly what csa2_select_topk returns for
 *            the pool and its scores, without a separate pass over them.
 *   sel_len  [B] int32 out when k > 0: min(k, P_eff).
 *   ws, ws_bytes: workspace of csa2_workspace_bytes(CSA2_OP_INDEX_FULL, B,
 *            max_len, total_len, H, P, k, ...) bytes, 256-byte aligned.  Its
 *            contents need no initialisation and are not preserved.
 * Requires Dk == 64, 1 <= H <= 64, 1 <= P, 0 <= k <= P, window >= 0.  Scores
 * are exact int32 (at most 64 * 15 * 64 * 127^2 < 2^31).  Ties at the pool
 * and selection boundaries go to the lower position.
 */
int csa2_index_full(const signed char* q, const signed char* w, const signed char* keys,
                    const long long* row_off, const int* len, int B, long long max_len,
                    long long total_len, int H, int Dk, int window, int P,
                    int* pool_pos, int* pool_score, int* pool_len,
                    int k, int* sel_pos, int* sel_len,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_index_score -- the scoring stage of csa2_index_full alone: the exact
 * index score of every eligible position p < E_b = max(len[b] - window, 0),
 *   score[b][p] = sum_h w[b][h] * max(0, q[b][h] . keys[row_off[b] + p]).
 * ("DeepSeek V4.1-Flash 552B runs like 16B (CED)", "Act 2": the indexer
 * scores the context with a small int8 query per head; the score is the
 * weighted sum of the per-head ReLU dot products.)
 *   q, w, keys, row_off, len, max_len, total_len, H, Dk, window: as
 *            csa2_index_full (window = 0 scores every cached position).
 *   score    [B][max_len] int32 out; entries p >= E_b are not written.
 *   ws, ws_bytes: as csa2_index_full (same size query, P ignored);
 *            no initialisation needed, contents not preserved.
 * Requires Dk == 64, 1 <= H <= 64, max_len <= 8,388,608.
 */
int csa2_index_score(const signed char* q, const signed char* w, const signed char* keys,
                     const long long* row_off, const int* len, int B, long long max_len,
                     long long total_len, int H, int Dk, int window, int* score,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_index_reindex -- Reindex mode: re-score only the candidate list with
 * this layer's own index query and weights, reading the same index keys.
 * ("DeepSeek V4.1-Flash 552B runs like 16B (CED)", "Act 2": later layers
 * search only that much smaller pool; "How DeepSeek V4.1 Flash Actually
 * Works", item 2: later layers search within that shortlist.)
 *   q, w, keys, row_off: as csa2_index_full.
 *   cand_pos [B][P] int32 positions (the Full layer's pool), cand_len [B].
 *   score    [B][P] int32 out: score of cand_pos[b][i] for i < cand_len[b],
 *            -1 for the rest.
 * Requires Dk == 64, 1 <= H <= 64, P >= 1.  No workspace.
 */
int csa2_index_reindex(const signed char* q, const signed char* w, const signed char* keys,
                       const long long* row_off, const int* cand_pos, const int* cand_len,
                       int B, int H, int Dk, int P, int* score, void* stream);

/*
 * csa2_select_topk -- keep the first k_eff = min(k, cand_len[b]) candidates
 * under the rank order (score descending, then lower position), output
 * ascending by position.
 * ("How DeepSeek V4.1 Flash Actually Works", item 2: the 512 most relevant
 * KV entries; "DeepSeek Has Done It Again...": up to 512 global positions.)
 *   score    [B][P] int32 (values >= 0 for valid entries).
 *   cand_pos [B][P] int32 positions, strictly ascending over the valid
 *            entries (as produced by csa2_index_full).
 *   sel_pos  [B][k] int32 out, ascending, tail -1;  sel_len [B] out.
 *   ws may be NULL when csa2_workspace_bytes(CSA2_OP_SELECT_TOPK, ...) is 0.
 * Requires 1 <= k <= P <= 16384.
 */
int csa2_select_topk(const int* score, const int* cand_pos, const int* cand_len,
                     int B, int P, int k, int* sel_pos, int* sel_len,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_sparse_attn_decode -- attention of every query head over
 * S_b = {sel_pos[b][0 .. sel_len[b])} U [L_b - min(window, L_b), L_b),
 * reading the FP4 latent cache of one layer (MQA, K = V = latent):
 *   out[b][h][:] = sum_j softmax_j(sm_scale * q[b][h] . v_j) v_j
 *   lse[b][h]    = ln sum_j exp(sm_scale * q[b][h] . v_j)
 * ("How DeepSeek V4.1 Flash Actually Works", item 2: the 512 selected
 * entries plus a local 128-token window; "DeepSeek Has Done It Again...":
 * up to 512 global positions alongside the most recent 128 tokens.)
 *   q_bf16   [B][Hq][D] bf16, 16-byte aligned.
 *   kv_fp4, kv_scale: this layer's cache (layout as csa2_kv_append_fp4).
 *   row_off, len, max_len: as csa2_index_full.
 *   sel_pos  [B][k] int32 selected positions (all < L_b - window), sel_len [B].
 *   out      [B][Hq][D] fp32;  lse [B][Hq] fp32 or NULL.
 *   ws, ws_bytes: workspace of csa2_workspace_bytes(CSA2_OP_SPARSE_ATTN, B,
 *            max_len, 0, 0, 0, k, Hq, D, window) bytes (split-K partials),
 *            256-byte aligned; no initialisation needed.
 * The selection is split across workgroups and the partial softmax states
 * are merged with a log-sum-exp combine, so fp32 results are deterministic
 * for a given (B, Hq, k, window).  A sequence with L_b == 0 gets out = 0 and
 * lse = -inf.  Requires D == 512, Hq a positive multiple of 16 (<= 1024), k >= 0,
 * k + window <= 16384.
 */
int csa2_sparse_attn_decode(const void* q_bf16, const unsigned char* kv_fp4,
                            const unsigned char* kv_scale, const long long* row_off,
                            const int* len, long long max_len, const int* sel_pos,
                            const int* sel_len, int B, int Hq, int D, int k, int window,
                            float sm_scale, float* out, float* lse,
                            void* ws, size_t ws_bytes, void* stream);


#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
