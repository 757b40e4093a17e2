/*
 * csa2.h -- C ABI of libcsa2.so: the decode hot path of CSA2 hierarchical
 * sparse attention on AMD MI355X (gfx950).
 *
 * What the path computes (page title, section):
 *  - "DeepSeek V4.1-Flash 552B runs like 16B (CED)", "Act 2: CSA2 &
 *    Hierarchical Sparse Indexing": one Full pass ranks the whole context
 *    into a candidate pool; Reindex layers rank that pool again, and Reuse
 *    layers keep the previous selection.
 *  - "How DeepSeek V4.1 Flash Actually Works", "The three KV-cache
 *    optimizations", item 2: each layer attends to 512 selected positions and
 *    the newest 128 tokens; the Full pass keeps at most 16,384 candidates;
 *    the KV cache holds 4-bit floating-point values.
 *  - "DeepSeek Has Done It Again...", "Architecture and inference efficiency":
 *    at most 512 positions from the history, next to the newest 128 tokens.
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
 * ("DeepSeek V4.1-Flash 552B runs like 16B (CED)", "Act 3", and "How
 * DeepSeek V4.1 Flash Actually Works", item 2: the KV cache is stored at 4
 * bits per value, down from 8.)
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
 * csa2_append_token -- one decode step's cache update: each sequence's new
 * token is written into the index-key cache and into every layer's FP4 KV
 * cache, and the sequence's length advances by one.  For sequence b, with
 * L = len[b] as stored on the device and row r = row_off[b] + L:
 *   keys[r][:]                      = key_rows[b][:]
 *   FP4 row l * layer_rows + r      = quantise(x_bf16[l][b][:])  for each layer l
 *   len[b]                          = L + 1
 * The quantisation is exactly that of csa2_kv_append_fp4.  The token is the
 * newest position of the sequence, so the layers that run afterwards attend
 * to it as part of the window.  Because the row follows from len on the
 * device, a captured step appends at the next position on every replay.
 * ("DeepSeek V4.1-Flash 552B runs like 16B (CED)", "Act 3": the main KV cache
 * is kept in 4-bit floating point; the order "write, then attend" is this
 * library's reading.)
 *   x_bf16   [n_layers][B][D] bf16, 16-byte aligned (may be NULL when n_layers == 0).
 *   key_rows [B][Dk] int8, 16-byte aligned.
 *   row_off  [B] int64 (device); len [B] int32 (device, read and advanced).
 *   layer_rows  rows per layer of kv_fp4 / kv_scale (layer l's row r is row
 *            l * layer_rows + r of the arrays).
 *   kv_fp4   [n_layers * layer_rows][D/2] uint8, 4-byte aligned;
 *   kv_scale [n_layers * layer_rows][D/32] uint8.
 *   keys     index-key cache [rows][Dk] int8, 16-byte aligned.
 * The caller guarantees that row row_off[b] + len[b] belongs to sequence b
 * (its reserved rows are not exhausted); the library does not check it.
 * Errors: INVALID for null pointers, negative sizes, D % 32 != 0 or a
 * misaligned pointer; UNSUPPORTED for Dk != 64 or B > 65535.  B == 0 is a
 * no-op.
 */
int csa2_append_token(const void* x_bf16, const signed char* key_rows,
                      const long long* row_off, int* len, int B, int n_layers,
                      long long layer_rows, int D, int Dk, unsigned char* kv_fp4,
                      unsigned char* kv_scale, signed char* keys, void* stream);

/*
 * csa2_append_tokens -- csa2_append_token for n tokens per sequence at once:
 * token j of sequence b goes to position len[b] + j (row row_off[b] + len[b]
 * + j), and len[b] advances by n.  A verify block appends its drafted tokens
 * with one call; a resumed session replays its dropped window with one call
 * (csa2_session_import).
 *   x_bf16   [n][n_layers][B][D] bf16 (token-major), 16-byte aligned.
 *   key_rows [n][B][Dk] int8, 16-byte aligned.
 *   row_off, len, layer_rows, D, Dk, kv_fp4, kv_scale, keys: as
 *            csa2_append_token.
 * A few rows per sequence are written by one workgroup per sequence; many
 * (a replayed window) by a grid of workgroups, then a second kernel writes
 * the index keys and advances len.  The caller guarantees that rows
 * row_off[b] + len[b] .. + n - 1 belong to sequence b.
 * Errors as csa2_append_token; n == 0 is a no-op.
 */
int csa2_append_tokens(const void* x_bf16, const signed char* key_rows,
                       const long long* row_off, int* len, int B, int n, int n_layers,
                       long long layer_rows, int D, int Dk, unsigned char* kv_fp4,
                       unsigned char* kv_scale, signed char* keys, void* stream);

/*
 * Sessions: what outlives a session, and its restore (bounded replay).
 * ("How DeepSeek V4.1 Flash Actually Works", "The three KV-cache
 * optimizations", item 3: the local state of the newest 128 tokens is kept
 * only during an active session and is rebuilt by replaying those tokens;
 * "DeepSeek V4.1-Flash 552B runs like 16B (CED)", "Act 3: FP4 KV & SWA
 * Bounded Replay".)  In this library a sequence's state is its index keys
 * and the FP4 rows of every layer.  csa2_session_export saves positions
 * [0, L - min(replay, L)) of each sequence; the newest min(replay, L)
 * positions are dropped.  csa2_session_import writes a saved state into the
 * caches (possibly at other rows) and sets len to the saved length; the
 * caller then appends the replayed tokens with csa2_append_tokens.  The
 * replay itself (recomputing those tokens' rows) needs the model and is not
 * part of this library.
 * Saved arrays (cap rows per sequence, cap >= the longest saved length):
 *   saved_keys  [B][cap][Dk] int8;
 *   saved_fp4   [n_layers][B][cap][D/2];  saved_scale [n_layers][B][cap][D/32];
 *   saved_len   [B] int32: positions saved per sequence.
 * Every array may be device memory or pinned host memory (hipHostMalloc);
 * the copy runs in a kernel on `stream`.  All data pointers 16-byte aligned.
 * Requires Dk == 64 and D a multiple of 512 (else UNSUPPORTED).  A sequence
 * with more than cap positions to save keeps only its first cap (saved_len
 * says how many).
 */
int csa2_session_export(const long long* row_off, const int* len, int B, int replay,
                        long long cap, int n_layers, long long layer_rows, int D, int Dk,
                        const unsigned char* kv_fp4, const unsigned char* kv_scale,
                        const signed char* keys, unsigned char* saved_fp4,
                        unsigned char* saved_scale, signed char* saved_keys, int* saved_len,
                        void* stream);

/* csa2_session_import -- inverse of csa2_session_export: rows [0,
 * saved_len[b]) of the saved arrays go to rows row_off[b] + p of the caches,
 * and len[b] = saved_len[b] (device).  Arguments as csa2_session_export. */
int csa2_session_import(const long long* row_off, int* len, const int* saved_len, int B,
                        long long cap, int n_layers, long long layer_rows, int D, int Dk,
                        const unsigned char* saved_fp4, const unsigned char* saved_scale,
                        const signed char* saved_keys, unsigned char* kv_fp4,
                        unsigned char* kv_scale, signed char* keys, void* stream);

/*
 * csa2_index_full -- Full mode: score every eligible position of each
 * sequence and keep the first P_eff = min(P, E_b) positions under the rank
 * order as the candidate pool.
 * ("DeepSeek V4.1-Flash 552B runs like 16B (CED)", "Act 2": one Full pass
 * over the context yields the pool the later indexing layers work from; "How
 * DeepSeek V4.1 Flash Actually Works", item 2: the pool holds at most 16,384
 * positions.)
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
 * ("DeepSeek V4.1-Flash 552B runs like 16B (CED)", "Act 2", and "How
 * DeepSeek V4.1 Flash Actually Works", item 2: a Reindex layer ranks the Full
 * layer's pool again rather than the whole context.)
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
 * ("How DeepSeek V4.1 Flash Actually Works", item 2, and "DeepSeek Has Done
 * It Again...", "Architecture and inference efficiency": a layer attends to a
 * selection of 512 positions from the history.)
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
 * ("How DeepSeek V4.1 Flash Actually Works", item 2, and "DeepSeek Has Done
 * It Again...", "Architecture and inference efficiency": a layer attends to
 * its 512 selected positions together with the newest 128 tokens.)
 *   q_bf16   [B][Hq][D] bf16, 16-byte aligned.
 *   kv_fp4, kv_scale: this layer's cache (layout as csa2_kv_append_fp4);
 *            kv_fp4 16-byte aligned (rows are read in 16-byte pieces),
 *            kv_scale 2-byte aligned.
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
 * Numeric range: every E8M0 scale byte 0..254 is read exactly (the rows are
 * dequantised relative to the largest scale byte among the rows a wave
 * holds, and that power of two is applied to the scores and outputs; a wave
 * whose scale bytes all lie in [2, 200] uses the absolute scales).  The
 * results meet 1e-3 * max|out| whenever every score sm_scale * q . v is
 * finite in fp32; blocks more than 126 octaves below the largest scale of
 * their workgroup's rows are taken as zero (their contribution is below
 * 2^-126 of the largest value).  Scale byte 255 (NaN in E8M0) is not valid
 * input; csa2_kv_append_fp4 never writes it.
 * Errors: INVALID for null pointers, negative sizes, Hq not a multiple of 16
 * or a misaligned pointer; UNSUPPORTED for D != 512 or k + window > 16384;
 * WORKSPACE for a missing or small workspace.
 */
int csa2_sparse_attn_decode(const void* q_bf16, const unsigned char* kv_fp4,
                            const unsigned char* kv_scale, const long long* row_off,
                            const int* len, long long max_len, const int* sel_pos,
                            const int* sel_len, int B, int Hq, int D, int k, int window,
                            float sm_scale, float* out, float* lse,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * Verify blocks.  A decode step may check several drafted tokens at once: the
 * T newest cached positions of a sequence (the last T tokens appended, all
 * counted in len[b], so len[b] >= T) form its block, and token t = 0 .. T-1
 * sits at position L_t - 1 with L_t = len[b] - (T - 1 - t).  (A sequence
 * shorter than its block is not valid input; the kernels give its tokens
 * with L_t <= 0 empty lists and attention output 0, lse -inf.)  Token t sees positions 0 .. L_t - 1
 * only: its window is [L_t - min(window, L_t), L_t) and its eligible positions
 * are [0, E_t), E_t = max(0, L_t - window).  Two selection modes:
 *  - per-token (shared == 0): every token has its own pool and selection,
 *    ranked by its own scores over its own eligible positions; list b * T + t
 *    of every [B][T][...] array below belongs to token t of sequence b;
 *  - shared (shared == 1): one pool and one selection per sequence,
 *    ranked by the best score over the block's tokens, max_t score_t(p), over
 *    the positions every token may rank, [0, E_0).  Each token still attends
 *    to its own window.
 * With T == 1 both modes are the one-token calls above.
 * ("DeepSeek Has Done It Again...", "Architecture and inference efficiency",
 * the DSpark bullet: the main model checks several drafted tokens together,
 * in blocks of five in the described set-up; "DeepSeek V4.1-Flash 552B runs
 * like 16B (CED)", "DSpark, Engram & Single-Pass mHC": several tokens can be
 * accepted in one step.  The pages do not say how the block's tokens share
 * the sparse selection; both readings are provided.)
 */

/* Workspace of a verify-block call: csa2_workspace_bytes with the sizes of a
 * block of T tokens per sequence.  CSA2_OP_SPARSE_ATTN and CSA2_OP_SELECT_TOPK
 * need what the one-token op needs for B * T query rows. */
size_t csa2_block_workspace_bytes(int op, int B, int T, int shared, long long max_len,
                                  long long total_len, int H, int P, int k, int Hq, int D,
                                  int window);

/*
 * csa2_index_full_block -- csa2_index_full for a verify block of T tokens per
 * sequence.  The index keys are read once for all T tokens.
 *   q        [B][T][H][Dk] int8 (token t's index query), 16-byte aligned.
 *   w        [B][T][H] int8 head weights in [0, 15].
 *   keys, row_off, len, max_len, total_len, H, Dk, window, P, k: as
 *            csa2_index_full (len counts every token of the block).
 *   shared   0: per-token lists; pool_pos / pool_score [B][T][P], pool_len
 *            [B][T], sel_pos [B][T][k], sel_len [B][T].
 *            1: one list per sequence; pool_pos / pool_score [B][P], pool_len
 *            [B], sel_pos [B][k], sel_len [B]; the scores are the block's best.
 *   ws, ws_bytes: csa2_block_workspace_bytes(CSA2_OP_INDEX_FULL, B, T, shared,
 *            max_len, total_len, H, P, k, ...) bytes, 256-byte aligned.
 * Requires 1 <= T <= 1024 (else UNSUPPORTED) and the csa2_index_full limits;
 * UNSUPPORTED when the call has more than 65535 lists.  A long block with
 * per-token lists is also the chunked form of prefill indexing: the C tokens
 * of a prompt chunk, appended to the cache, each rank their own causal prefix
 * in one call.
 * ("DeepSeek V4.1-Flash 552B runs like 16B (CED)", "Act 1: Causal
 * Encoder-Decoder", and "How DeepSeek V4.1 Flash Actually Works", item 1:
 * prompt tokens go through the lower layers to build the global cache, so a
 * prompt is indexed many query tokens at a time.)
 */
int csa2_index_full_block(const signed char* q, const signed char* w, const signed char* keys,
                          const long long* row_off, const int* len, int B, int T, int shared,
                          long long max_len, long long total_len, int H, int Dk, int window,
                          int P, int* pool_pos, int* pool_score, int* pool_len, int k,
                          int* sel_pos, int* sel_len, void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_index_score_block -- the scoring stage of csa2_index_full_block alone.
 *   q, w, keys, row_off, len, B, T, shared, max_len, total_len, H, Dk,
 *            window: as csa2_index_full_block.
 *   score    shared == 0: [B][T][max_len] int32 out, score[b][t][p] = token
 *            t's score of position p for p < E_t (later entries not written);
 *            shared == 1: [B][max_len], the best score over the block's tokens
 *            for p < E_0.
 *   ws, ws_bytes: as csa2_index_full_block with k = 0.
 */
int csa2_index_score_block(const signed char* q, const signed char* w, const signed char* keys,
                           const long long* row_off, const int* len, int B, int T, int shared,
                           long long max_len, long long total_len, int H, int Dk, int window,
                           int* score, void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_index_reindex_block -- csa2_index_reindex for a verify block.
 *   q [B][T][H][Dk], w [B][T][H]: as csa2_index_full_block.
 *   shared   0: cand_pos / score [B][T][P], cand_len [B][T]; list b * T + t
 *            is scored with token t's query.
 *            1: cand_pos / score [B][P], cand_len [B]; each candidate gets the
 *            best score over the block's tokens.
 * Requires T >= 1 and the csa2_index_reindex limits; UNSUPPORTED when the call
 * has more than 65535 lists.  No workspace.
 */
int csa2_index_reindex_block(const signed char* q, const signed char* w, const signed char* keys,
                             const long long* row_off, const int* cand_pos, const int* cand_len,
                             int B, int T, int shared, int H, int Dk, int P, int* score,
                             void* stream);

/*
 * csa2_sparse_attn_decode_block -- csa2_sparse_attn_decode for a verify
 * block: token t of sequence b attends to its selection and to its own
 * window [L_t - min(window, L_t), L_t).
 *   q_bf16   [B][T][Hq][D] bf16;  out [B][T][Hq][D] fp32;  lse [B][T][Hq] or NULL.
 *   shared   0: sel_pos [B][T][k], sel_len [B][T] (token t's own selection);
 *            1: sel_pos [B][k], sel_len [B] (one selection for the block; its
 *            positions must be < E_0 so that no token attends a position twice).
 *   ws, ws_bytes: csa2_block_workspace_bytes(CSA2_OP_SPARSE_ATTN, B, T, shared,
 *            max_len, 0, 0, 0, k, Hq, D, window) bytes.
 * Same numerics, limits and errors as csa2_sparse_attn_decode, with B * T
 * query rows (UNSUPPORTED for T > 1024 or B * T > 65535).
 */
int csa2_sparse_attn_decode_block(const void* q_bf16, const unsigned char* kv_fp4,
                                  const unsigned char* kv_scale, const long long* row_off,
                                  const int* len, long long max_len, const int* sel_pos,
                                  const int* sel_len, int B, int T, int shared, int Hq, int D,
                                  int k, int window, float sm_scale, float* out, float* lse,
                                  void* ws, size_t ws_bytes, void* stream);

/* Bytes of device scratch behind csa2_sparse_attn_decode_static (per GPU). */
#define CSA2_ATTN_STATIC_SCRATCH_BYTES (32u << 20)

/*
 * csa2_sparse_attn_decode_static -- csa2_sparse_attn_decode for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The arguments and results are those
 * of csa2_sparse_attn_decode without ws / ws_bytes (the same kernels run); the
 * split-K partials go to a scratch array of CSA2_ATTN_STATIC_SCRATCH_BYTES
 * (32 MiB) that the library keeps in device memory, one per GPU, from the
 * library's first use on that GPU until the process ends.  The call allocates
 * nothing (no hipMalloc, no allocating library routine).
 *  - Sizes whose partials need more than that
 *    (csa2_workspace_bytes(CSA2_OP_SPARSE_ATTN, ...) > 32 MiB, e.g. more than
 *    about 50 sequences of 64 heads with k = 512 and window 128) are rejected
 *    with CSA2_ERR_UNSUPPORTED and nothing is launched.
 *  - `stream` must belong to the current device (else CSA2_ERR_INVALID).
 *  - Every call on one GPU uses that GPU's one scratch array: calls that
 *    overlap in time on one GPU (streams not ordered with each other) race and
 *    their results are undefined.  Calls ordered on one stream are safe.  The
 *    scratch needs no initialisation; it keeps the last call's partials.
 */
int csa2_sparse_attn_decode_static(const void* q_bf16, const unsigned char* kv_fp4,
                                   const unsigned char* kv_scale, const long long* row_off,
                                   const int* len, long long max_len, const int* sel_pos,
                                   const int* sel_len, int B, int Hq, int D, int k, int window,
                                   float sm_scale, float* out, float* lse, void* stream);


#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
