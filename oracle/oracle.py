"""Plain CPU oracle for the CSA2 hierarchical sparse-attention decode step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark import this module; the product path never does, and it
shares no code, table or helper with the HIP kernels.

The heavy loops live in ``csa2_oracle.c`` (plain C, int64 / fp64, built with
gcc); this file is the literal orchestration of the method in numpy, one
function per step of the method, each naming the passage it follows.

Sources (page title, section):
  [CED]  "DeepSeek V4.1-Flash 552B runs like 16B (CED)", "Act 2: CSA2 &
         Hierarchical Sparse Indexing" and "Act 3: FP4 KV & SWA Bounded Replay".
  [HOW]  "How DeepSeek V4.1 Flash Actually Works", "The three KV-cache
         optimizations", item 2 "Compress Sparse Attention".
  [AGAIN] "DeepSeek Has Done It Again...", "Architecture and inference
         efficiency", bullet "Sparse attention for long context".
  [IMP]  "Deepseek just did the impossible", "Memory and Compute Optimization".
Readings fixed where the pages are silent (int8 keys/queries, the score rule,
tie order, FP4 E2M1 + E8M0 per 32, K = V = latent, 1/sqrt(512)) are listed with
each function.

Parity status: all functions are pinned by the CPU tests; none is unpinned.
The multi-token block functions at the end are pinned against the single-
token step (T = 1), plain-Python scores with exhaustive ranking, causality
and dense causal softmax attention.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa2_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libcsa2_oracle.so")

__all__ = [
    "build", "load", "bf16_to_f64", "fp4_quantize", "fp4_dequantize", "fp4_value",
    "index_scores", "topk", "eligible_count", "window_positions", "index_full",
    "index_reindex", "select_topk", "attention_positions", "attention",
    "layer_kind", "layer_pattern", "decode_step", "block_lengths", "index_full_block",
    "index_reindex_block", "decode_block", "session_saved_length", "session_export",
    "session_import", "replay_append",
]


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into a shared object next to the source."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                        _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None

# A test may point the loader at another build of the same source (for
# example one compiled with the address and undefined-behaviour sanitizers).
_LIB_ENV = "CSA2_ORACLE_LIB"


def load():
    global _lib
    if _lib is None:
        path = os.environ.get(_LIB_ENV)
        if not path:
            path = _LIB_PATH
            if not os.path.exists(_LIB_PATH) or \
                    os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build(force=True)
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        lib.oracle_fp4_value.argtypes = [ctypes.c_int, ctypes.c_int]
        lib.oracle_fp4_value.restype = ctypes.c_double
        lib.oracle_fp4_quantize.argtypes = [P, I64, ctypes.c_int, P, P]
        lib.oracle_fp4_quantize.restype = None
        lib.oracle_fp4_dequantize.argtypes = [P, P, I64, ctypes.c_int, P]
        lib.oracle_fp4_dequantize.restype = None
        lib.oracle_index_scores.argtypes = [P, ctypes.c_int, P, I64, P, P, ctypes.c_int, P]
        lib.oracle_index_scores.restype = None
        lib.oracle_topk.argtypes = [P, P, I64, I64, P, P]
        lib.oracle_topk.restype = I64
        lib.oracle_attention.argtypes = [P, ctypes.c_int, ctypes.c_int, P, I64,
                                         ctypes.c_double, P, P]
        lib.oracle_attention.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------
# FP4 E2M1 with one E8M0 scale per 32 elements ([CED] "Act 3": FP4 main KV;
# [HOW] item 2: KV values stored in FP4; block format per OCP MX v1.0).
# --------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def fp4_value(nibble: int, scale_byte: int) -> float:
    return load().oracle_fp4_value(int(nibble), int(scale_byte))


def fp4_quantize(x_bf16: np.ndarray):
    """Rows of D bf16 values (uint16 bit patterns, shape [n, D]) ->
    (codes [n, D/2] uint8, scales [n, D/32] uint8)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    n, D = x.shape
    assert D % 32 == 0
    codes = np.zeros((n, D // 2), dtype=np.uint8)
    scales = np.zeros((n, D // 32), dtype=np.uint8)
    if n:
        load().oracle_fp4_quantize(_ptr(x), n, D, _ptr(codes), _ptr(scales))
    return codes, scales


def fp4_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.uint8)
    n, half = c.shape
    D = half * 2
    assert s.shape == (n, D // 32)
    out = np.zeros((n, D), dtype=np.float64)
    if n:
        load().oracle_fp4_dequantize(_ptr(c), _ptr(s), n, D, _ptr(out))
    return out


# --------------------------------------------------------------------------
# Index scores and the rank order.
# --------------------------------------------------------------------------

_SCORE_LIMIT = 1 << 31


def index_scores(keys: np.ndarray, rows: np.ndarray, q: np.ndarray, w: np.ndarray) -> np.ndarray:
    """s(p) = sum_h w_h * max(0, q_h . K[p]) for every listed cache row.

    The pages say an indexing layer scans the context and scores positions
    ([HOW] item 2; [CED] "Act 2"); the rule itself (int8 keys and queries, one
    key per token shared by all index heads, per-head weights, ReLU, exact
    integer sum) is this path's reading.  Returned as int64; every value is
    asserted to lie in [0, 2^31).
    """
    keys = np.ascontiguousarray(keys, dtype=np.int8)
    dk = keys.shape[1]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    q = np.ascontiguousarray(q, dtype=np.int8)
    w = np.ascontiguousarray(w, dtype=np.int8)
    H = q.shape[0]
    assert q.shape == (H, dk) and w.shape == (H,)
    out = np.zeros(rows.shape[0], dtype=np.int64)
    if rows.shape[0]:
        assert rows.min() >= 0 and rows.max() < keys.shape[0]
        load().oracle_index_scores(_ptr(keys), dk, _ptr(rows), rows.shape[0],
                                   _ptr(q), _ptr(w), H, _ptr(out))
        assert out.min() >= 0 and out.max() < _SCORE_LIMIT
    return out


def topk(score: np.ndarray, pos: np.ndarray, k: int):
    """The first min(k, n) candidates under the order  p before p'  iff
    s(p) > s(p') or (s(p) == s(p') and p < p'), returned ascending by
    position together with their scores.

    [HOW] item 2 and [AGAIN]: a layer keeps a selection of 512 positions;
    ties go to the lower position (this path's reading).
    """
    s = np.ascontiguousarray(score, dtype=np.int64)
    p = np.ascontiguousarray(pos, dtype=np.int64)
    n = s.shape[0]
    assert p.shape == (n,)
    keff = max(0, min(int(k), n))
    out_p = np.zeros(keff, dtype=np.int64)
    out_s = np.zeros(keff, dtype=np.int64)
    if keff:
        got = load().oracle_topk(_ptr(s), _ptr(p), n, keff, _ptr(out_p), _ptr(out_s))
        assert got == keff
    return out_p, out_s


# --------------------------------------------------------------------------
# The CSA2 modes.
# --------------------------------------------------------------------------

def eligible_count(L: int, window: int) -> int:
    """Positions eligible for global selection: [0, L - W).  The window rows
    [L - W, L) are attended anyway and are never selected twice ([HOW] item 2:
    the selection and the newest 128 tokens are attended side by side)."""
    return max(0, int(L) - int(window))


def window_positions(L: int, window: int) -> np.ndarray:
    return np.arange(max(0, int(L) - int(window)), int(L), dtype=np.int64)


def index_full(keys, row_off: int, L: int, q, w, window: int, P: int):
    """Full mode: score every eligible position of the context and keep the
    first min(P, E) under the rank order as the candidate pool, ascending by
    position ([CED] "Act 2": one Full pass over the context yields the pool
    the later layers work from; [HOW] item 2: at most 16,384 positions)."""
    E = eligible_count(L, window)
    pos = np.arange(E, dtype=np.int64)
    s = index_scores(keys, row_off + pos, q, w)
    return topk(s, pos, min(int(P), E))


def index_reindex(keys, row_off: int, cand_pos, q, w) -> np.ndarray:
    """Reindex mode: re-score only the pool with this layer's own index query
    and weights and the same index keys ([CED] "Act 2" and [HOW] item 2: a
    Reindex layer ranks the Full layer's pool again, not the context)."""
    cand_pos = np.asarray(cand_pos, dtype=np.int64)
    return index_scores(keys, row_off + cand_pos, q, w)


def select_topk(score, cand_pos, k: int):
    """Top-k global positions of a scored candidate list, ascending by position
    ([HOW] item 2: a layer's selection of 512 positions)."""
    return topk(score, cand_pos, k)


def attention_positions(L: int, sel_pos, window: int) -> np.ndarray:
    """S = selection U window, selection first; the two are disjoint."""
    sel = np.asarray(sel_pos, dtype=np.int64)
    win = window_positions(L, window)
    assert sel.size == 0 or sel.max() < max(0, L - window), "selection overlaps the window"
    return np.concatenate([sel, win])


def attention(q_bf16: np.ndarray, codes: np.ndarray, scales: np.ndarray, sm_scale: float):
    """Softmax attention of every query head over the given FP4 rows, K = V =
    the dequantised latent row (MQA).  Returns (out [Hq, D] float64,
    lse [Hq] float64, natural log).  [HOW] item 2 / [AGAIN]: attention over the
    selected global positions and the recent window."""
    v = fp4_dequantize(codes, scales)
    q = np.ascontiguousarray(q_bf16, dtype=np.uint16)
    Hq, D = q.shape
    S = v.shape[0]
    assert v.shape[1] == D
    out = np.zeros((Hq, D), dtype=np.float64)
    lse = np.zeros(Hq, dtype=np.float64)
    load().oracle_attention(_ptr(q), Hq, D, _ptr(np.ascontiguousarray(v)), S,
                            float(sm_scale), _ptr(out), _ptr(lse))
    return out, lse


def layer_kind(l: int) -> str:
    """Layer pattern of the 20-layer decoder: Full once, then Reindex at layer 1
    and every 4th layer, Reuse otherwise ([CED] "Act 2": Full -> Reindex ->
    Reuse; [IMP]: Full, Reindex and Reuse sharing modes)."""
    if l == 0:
        return "F"
    if l == 1 or l % 4 == 0:
        return "R"
    return "U"


def layer_pattern(n_layers: int) -> str:
    return "".join(layer_kind(l) for l in range(n_layers))


def decode_step(pattern: str, keys, row_off: int, L: int, window: int, P: int, k: int,
                idx_q, idx_w, attn_q, kv_rows, sm_scale: float):
    """One decode step of one sequence over the layers of ``pattern``.

    idx_q[l], idx_w[l]: int8 index query / weights of F and R layers.
    attn_q[l]: [Hq, D] bf16 bit patterns.  kv_rows(l, positions) -> bf16 bit
    patterns [n, D] of layer l's latent rows at those positions (quantised
    here with the oracle's own FP4 rule).
    Returns per-layer dicts with pool, selection, out and lse.
    Reuse takes the most recent layer's selection; Reindex re-scores the most
    recent Full layer's pool ([CED] "Act 2"; [HOW] item 2: Reuse layers keep
    the selection of the layer before).
    """
    results = []
    pool = None
    sel = None
    for l, kind in enumerate(pattern):
        rec = {"kind": kind}
        if kind == "F":
            pool_pos, pool_score = index_full(keys, row_off, L, idx_q[l], idx_w[l], window, P)
            pool = pool_pos
            sel, _ = select_topk(pool_score, pool_pos, k)
            rec.update(pool_pos=pool_pos, pool_score=pool_score)
        elif kind == "R":
            assert pool is not None, "Reindex needs an earlier Full layer"
            sc = index_reindex(keys, row_off, pool, idx_q[l], idx_w[l])
            sel, _ = select_topk(sc, pool, k)
            rec.update(reindex_score=sc)
        else:
            assert sel is not None, "Reuse needs an earlier selection"
        S = attention_positions(L, sel, window)
        x = kv_rows(l, S)
        codes, scales = fp4_quantize(x)
        out, lse = attention(attn_q[l], codes, scales, sm_scale)
        rec.update(sel=sel, out=out, lse=lse, S=S)
        results.append(rec)
    return results


# --------------------------------------------------------------------------
# Multi-token decode: a block of T tokens verified in one step ("DeepSeek Has
# Done It Again...", "Architecture and inference efficiency", bullet on
# DSpark: drafted tokens are checked by the main model together, in blocks
# of five; "DeepSeek V4.1-Flash 552B runs like 16B (CED)", "DSpark, Engram &
# Single-Pass mHC").  Readings of this path, where the pages are silent:
#  * the block's T tokens are the last T cached positions; token t sits at
#    position L - T + t and sees positions 0 .. L - T + t only (causal), so
#    its own window is the 128 positions ending at itself;
#  * per-token selection: every token ranks its own eligible positions with
#    its own index query, exactly as a single decoding token would;
#  * shared selection: one pool and one selection for the block, ranking the
#    positions eligible for every token of the block (those of token 0) by the
#    best score any of the block's tokens gives them, max_t s_t(p); the
#    maximum stays an exact int32 (a sum of five scores would not).
# --------------------------------------------------------------------------

def block_lengths(L: int, T: int):
    """Cached positions seen by each token of a block of T tokens at the end
    of a context of L positions (the block included)."""
    assert 1 <= T <= L
    return [int(L) - int(T) + 1 + t for t in range(int(T))]


def _block_scores(keys, row_off: int, pos, q, w):
    """max over the block's tokens of each token's score at `pos`."""
    s = None
    for t in range(len(q)):
        st = index_scores(keys, row_off + np.asarray(pos, dtype=np.int64), q[t], w[t])
        s = st if s is None else np.maximum(s, st)
    return s


def index_full_block(keys, row_off: int, L: int, T: int, q, w, window: int, P: int, shared: bool):
    """Full mode for a block.  q: [T][H][Dk] int8, w: [T][H].  Per token: a list
    of T (pool_pos, pool_score), token t's pool over its own eligible positions.
    Shared: one (pool_pos, pool_score) over token 0's eligible positions,
    ranked by max_t s_t(p)."""
    Ls = block_lengths(L, T)
    if not shared:
        return [index_full(keys, row_off, Ls[t], q[t], w[t], window, P) for t in range(T)]
    E0 = eligible_count(Ls[0], window)
    pos = np.arange(E0, dtype=np.int64)
    return topk(_block_scores(keys, row_off, pos, q, w), pos, min(int(P), E0))


def index_reindex_block(keys, row_off: int, cand_pos, q, w, shared: bool):
    """Reindex for a block: per token, token t's own pool re-scored with its
    own query (cand_pos is then a list of T pools); shared, the block's pool
    re-scored with max_t s_t(p)."""
    if not shared:
        return [index_reindex(keys, row_off, cand_pos[t], q[t], w[t]) for t in range(len(q))]
    return _block_scores(keys, row_off, cand_pos, q, w)


def decode_block(pattern: str, keys, row_off: int, L: int, T: int, window: int, P: int, k: int,
                 idx_q, idx_w, attn_q, kv_rows, sm_scale: float, shared: bool):
    """One verify step of a block of T tokens of one sequence over the layers
    of ``pattern`` (Full, Reindex, Reuse as in decode_step).

    idx_q[l], idx_w[l]: [T][H][Dk] / [T][H] int8 of F and R layers.
    attn_q[l]: [T][Hq][D] bf16 bit patterns.  kv_rows(l, positions) as in
    decode_step.  Returns per layer a dict with the pool(s), the selection(s)
    (a list of T, or one shared), and per token out, lse and S.
    """
    Ls = block_lengths(L, T)
    results = []
    pool = None
    sel = None
    for l, kind in enumerate(pattern):
        rec = {"kind": kind}
        if kind == "F":
            res = index_full_block(keys, row_off, L, T, idx_q[l], idx_w[l], window, P, shared)
            if shared:
                pool, pool_score = res
                sel, _ = select_topk(pool_score, pool, k)
            else:
                pool = [r[0] for r in res]
                pool_score = [r[1] for r in res]
                sel = [select_topk(pool_score[t], pool[t], k)[0] for t in range(T)]
            rec.update(pool_pos=pool, pool_score=pool_score)
        elif kind == "R":
            assert pool is not None, "Reindex needs an earlier Full layer"
            sc = index_reindex_block(keys, row_off, pool, idx_q[l], idx_w[l], shared)
            if shared:
                sel, _ = select_topk(sc, pool, k)
            else:
                sel = [select_topk(sc[t], pool[t], k)[0] for t in range(T)]
            rec.update(reindex_score=sc)
        else:
            assert sel is not None, "Reuse needs an earlier selection"
        outs, lses, Ss = [], [], []
        for t in range(T):
            S = attention_positions(Ls[t], sel if shared else sel[t], window)
            codes, scales = fp4_quantize(kv_rows(l, S))
            out, lse = attention(attn_q[l][t], codes, scales, sm_scale)
            outs.append(out)
            lses.append(lse)
            Ss.append(S)
        rec.update(sel=sel, out=outs, lse=lses, S=Ss)
        results.append(rec)
    return results


# --------------------------------------------------------------------------
# Sessions and bounded replay ("How DeepSeek V4.1 Flash Actually Works", "The
# three KV-cache optimizations", item 3; "DeepSeek V4.1-Flash 552B runs like
# 16B (CED)", "Act 3: FP4 KV & SWA Bounded Replay").  Reading: a sequence's
# state is its index keys and the FP4 rows of every layer; what outlives a
# session is positions [0, L - min(R, L)) with R = 128 (the local window);
# the newest min(R, L) positions are dropped and come back by appending the
# replayed tokens, which the model recomputes.
# --------------------------------------------------------------------------

def session_saved_length(L: int, replay: int) -> int:
    """Positions of a sequence of length L that outlive its session."""
    return max(0, int(L) - min(int(replay), max(int(L), 0)))


def session_export(keys, fp4, scales, row_off: int, L: int, replay: int):
    """The saved state of one sequence: (n, keys[:n], [fp4_l[:n]], [scale_l[:n]])
    with n = session_saved_length(L, replay).  fp4 / scales: one array of rows
    per layer."""
    n = session_saved_length(L, replay)
    r = slice(int(row_off), int(row_off) + n)
    return n, keys[r].copy(), [f[r].copy() for f in fp4], [c[r].copy() for c in scales]


def session_import(saved, keys, fp4, scales, row_off: int) -> int:
    """Write a saved state into the caches at row_off; returns the new length."""
    n, k, f, c = saved
    r = slice(int(row_off), int(row_off) + n)
    keys[r] = k
    for dst, src in zip(fp4, f):
        dst[r] = src
    for dst, src in zip(scales, c):
        dst[r] = src
    return n


def replay_append(keys, fp4, scales, row_off: int, L: int, key_rows, x_bf16_rows):
    """Append replayed tokens at positions L, L + 1, ...: their index keys
    ([n][Dk]) and, per layer, their latent rows ([n][D] bf16, quantised with
    the FP4 rule).  Returns the new length."""
    n = len(key_rows)
    r = slice(int(row_off) + int(L), int(row_off) + int(L) + n)
    keys[r] = key_rows
    for l in range(len(fp4)):
        codes, sc = fp4_quantize(np.asarray(x_bf16_rows[l]))
        fp4[l][r] = codes
        scales[l][r] = sc
    return int(L) + n
