"""ctypes binding of libcsa2.so, same names as the C ABI (include/csa2.h).

Argument marshalling only: torch tensors give device pointers and the HIP
stream; every step of the decode path runs in the library's kernels.  The
library must have been built (``python -m decode_kv_amd.build``); nothing
here falls back to another implementation.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcsa2.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "csa2.h")
HEADERS = [HEADER, os.path.join(os.path.dirname(HERE), "include", "csa2_measure.h")]

CSA2_OK = 0
CSA2_ERR_INVALID = -1
CSA2_ERR_WORKSPACE = -2
CSA2_ERR_UNSUPPORTED = -3
CSA2_ERR_HIP = -4

OP_INDEX_FULL = 1
OP_SELECT_TOPK = 2
OP_SPARSE_ATTN = 3


class Csa2Error(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__("%s failed (%d): %s" % (fn, code, msg))
        self.code = code


_lib = None


def lib():
    """Load libcsa2.so (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libcsa2.so is not built; run `python -m decode_kv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        V, I, LL, SZ, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_size_t, ctypes.c_float
        L.csa2_last_error.restype = ctypes.c_char_p
        L.csa2_last_error.argtypes = []
        L.csa2_version.restype = ctypes.c_char_p
        L.csa2_version.argtypes = []
        L.csa2_workspace_bytes.restype = SZ
        L.csa2_workspace_bytes.argtypes = [I, I, LL, LL, I, I, I, I, I, I]
        L.csa2_kv_append_fp4.restype = I
        L.csa2_kv_append_fp4.argtypes = [V, V, I, I, V, V, V]
        L.csa2_append_token.restype = I
        L.csa2_append_token.argtypes = [V, V, V, V, I, I, LL, I, I, V, V, V, V]
        L.csa2_index_full.restype = I
        L.csa2_index_full.argtypes = [V, V, V, V, V, I, LL, LL, I, I, I, I, V, V, V, I, V, V, V, SZ,
                                       V]
        L.csa2_index_score.restype = I
        L.csa2_index_score.argtypes = [V, V, V, V, V, I, LL, LL, I, I, I, V, V, SZ, V]
        L.csa2_index_reindex.restype = I
        L.csa2_index_reindex.argtypes = [V, V, V, V, V, V, I, I, I, I, V, V]
        L.csa2_select_topk.restype = I
        L.csa2_select_topk.argtypes = [V, V, V, I, I, I, V, V, V, SZ, V]
        L.csa2_stream_read_sink_words.restype = SZ
        L.csa2_stream_read_sink_words.argtypes = [SZ]
        L.csa2_stream_read.restype = I
        L.csa2_stream_read.argtypes = [V, SZ, V, SZ, V]
        L.csa2_empty_kernel.restype = I
        L.csa2_empty_kernel.argtypes = [V]
        L.csa2_handoff_scratch_bytes.restype = SZ
        L.csa2_handoff_scratch_bytes.argtypes = [I, I]
        L.csa2_handoff.restype = I
        L.csa2_handoff.argtypes = [I, I, I, F, V, SZ, V, V]
        L.csa2_sparse_attn_decode_static.restype = I
        L.csa2_sparse_attn_decode_static.argtypes = [V, V, V, V, V, LL, V, V, I, I, I, I, I, F,
                                                     V, V, V]
        L.csa2_sparse_attn_decode.restype = I
        L.csa2_sparse_attn_decode.argtypes = [V, V, V, V, V, LL, V, V, I, I, I, I, I, F, V, V,
                                              V, SZ, V]
        L.csa2_append_tokens.restype = I
        L.csa2_append_tokens.argtypes = [V, V, V, V, I, I, I, LL, I, I, V, V, V, V]
        L.csa2_session_export.restype = I
        L.csa2_session_export.argtypes = [V, V, I, I, LL, I, LL, I, I, V, V, V, V, V, V, V, V]
        L.csa2_session_import.restype = I
        L.csa2_session_import.argtypes = [V, V, V, I, LL, I, LL, I, I, V, V, V, V, V, V, V]
        L.csa2_block_workspace_bytes.restype = SZ
        L.csa2_block_workspace_bytes.argtypes = [I, I, I, I, LL, LL, I, I, I, I, I, I]
        L.csa2_index_full_block.restype = I
        L.csa2_index_full_block.argtypes = [V, V, V, V, V, I, I, I, LL, LL, I, I, I, I, V, V, V,
                                            I, V, V, V, SZ, V]
        L.csa2_index_score_block.restype = I
        L.csa2_index_score_block.argtypes = [V, V, V, V, V, I, I, I, LL, LL, I, I, I, V, V, SZ, V]
        L.csa2_index_reindex_block.restype = I
        L.csa2_index_reindex_block.argtypes = [V, V, V, V, V, V, I, I, I, I, I, I, V, V]
        L.csa2_sparse_attn_decode_block.restype = I
        L.csa2_sparse_attn_decode_block.argtypes = [V, V, V, V, V, LL, V, V, I, I, I, I, I, I, I,
                                                    F, V, V, V, SZ, V]
        _lib = L
    return _lib


def header_source() -> str:
    """The declarations of include/csa2.h and include/csa2_measure.h, comments removed."""
    src = "".join(open(h).read() for h in HEADERS)
    return re.sub(r"/\*.*?\*/", "", src, flags=re.S)


def header_functions() -> list:
    """Names of the functions the headers declare."""
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", header_source())))


def last_error() -> str:
    return lib().csa2_last_error().decode()


def version() -> str:
    return lib().csa2_version().decode()


def _check(fn: str, rc: int):
    if rc != CSA2_OK:
        raise Csa2Error(fn, rc, last_error())


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _s(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def workspace_bytes(op: int, B: int, max_len: int = 0, total_len: int = 0, H: int = 0,
                    P: int = 0, k: int = 0, Hq: int = 0, D: int = 0, window: int = 0) -> int:
    return int(lib().csa2_workspace_bytes(op, B, max_len, total_len, H, P, k, Hq, D, window))


def workspace(nbytes: int, device="cuda"):
    """A 256-byte aligned device buffer (torch's allocator aligns to 512)."""
    if nbytes <= 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def kv_append_fp4(x_bf16, dst_row, kv_fp4, kv_scale, stream=None):
    n, D = x_bf16.shape
    _check("csa2_kv_append_fp4",
           lib().csa2_kv_append_fp4(_p(x_bf16), _p(dst_row), n, D, _p(kv_fp4), _p(kv_scale),
                                    _s(stream)))


def append_token(x_bf16, key_rows, row_off, lens, kv_fp4, kv_scale, keys, stream=None):
    """x_bf16 [n_layers][B][D]; kv_fp4 [n_layers][rows][D/2]; kv_scale
    [n_layers][rows][D/32]; key_rows [B][Dk]; keys [rows][Dk]."""
    n_layers, B, D = x_bf16.shape
    layer_rows = kv_fp4.shape[1]
    assert kv_fp4.shape[0] == n_layers and kv_scale.shape[:2] == kv_fp4.shape[:2]
    _check("csa2_append_token",
           lib().csa2_append_token(_p(x_bf16), _p(key_rows), _p(row_off), _p(lens), B, n_layers,
                                   layer_rows, D, key_rows.shape[1], _p(kv_fp4), _p(kv_scale),
                                   _p(keys), _s(stream)))


def append_tokens(x_bf16, key_rows, row_off, lens, kv_fp4, kv_scale, keys, stream=None):
    """x_bf16 [n][n_layers][B][D]; key_rows [n][B][Dk]; caches as append_token."""
    n, n_layers, B, D = x_bf16.shape
    layer_rows = kv_fp4.shape[1]
    assert kv_fp4.shape[0] == n_layers and kv_scale.shape[:2] == kv_fp4.shape[:2]
    _check("csa2_append_tokens",
           lib().csa2_append_tokens(_p(x_bf16), _p(key_rows), _p(row_off), _p(lens), B, n,
                                    n_layers, layer_rows, D, key_rows.shape[2], _p(kv_fp4),
                                    _p(kv_scale), _p(keys), _s(stream)))


def session_export(row_off, lens, replay, kv_fp4, kv_scale, keys, saved_fp4, saved_scale,
                   saved_keys, saved_len, stream=None):
    """Caches kv_fp4 [n_layers][rows][D/2], kv_scale [n_layers][rows][D/32],
    keys [rows][Dk]; saved arrays [n_layers][B][cap][...] and [B][cap][Dk]."""
    n_layers, layer_rows, half = kv_fp4.shape
    B, cap, Dk = saved_keys.shape
    _check("csa2_session_export",
           lib().csa2_session_export(_p(row_off), _p(lens), B, int(replay), cap, n_layers,
                                     layer_rows, 2 * half, Dk, _p(kv_fp4), _p(kv_scale), _p(keys),
                                     _p(saved_fp4), _p(saved_scale), _p(saved_keys),
                                     _p(saved_len), _s(stream)))


def session_import(row_off, lens, saved_len, saved_fp4, saved_scale, saved_keys, kv_fp4,
                   kv_scale, keys, stream=None):
    n_layers, layer_rows, half = kv_fp4.shape
    B, cap, Dk = saved_keys.shape
    _check("csa2_session_import",
           lib().csa2_session_import(_p(row_off), _p(lens), _p(saved_len), B, cap, n_layers,
                                     layer_rows, 2 * half, Dk, _p(saved_fp4), _p(saved_scale),
                                     _p(saved_keys), _p(kv_fp4), _p(kv_scale), _p(keys),
                                     _s(stream)))


def index_full(q, w, keys, row_off, lens, max_len, total_len, window, P, pool_pos, pool_score,
               pool_len, ws, stream=None, k=0, sel_pos=None, sel_len=None):
    B, H, Dk = q.shape
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("csa2_index_full",
           lib().csa2_index_full(_p(q), _p(w), _p(keys), _p(row_off), _p(lens), B, int(max_len),
                                 int(total_len), H, Dk, window, P, _p(pool_pos), _p(pool_score),
                                 _p(pool_len), int(k), _p(sel_pos), _p(sel_len), _p(ws), nbytes,
                                 _s(stream)))


def index_score(q, w, keys, row_off, lens, max_len, total_len, window, score, ws, stream=None):
    B, H, Dk = q.shape
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("csa2_index_score",
           lib().csa2_index_score(_p(q), _p(w), _p(keys), _p(row_off), _p(lens), B, int(max_len),
                                  int(total_len), H, Dk, window, _p(score), _p(ws), nbytes,
                                  _s(stream)))


def index_reindex(q, w, keys, row_off, cand_pos, cand_len, score, stream=None):
    B, H, Dk = q.shape
    P = cand_pos.shape[1]
    _check("csa2_index_reindex",
           lib().csa2_index_reindex(_p(q), _p(w), _p(keys), _p(row_off), _p(cand_pos),
                                    _p(cand_len), B, H, Dk, P, _p(score), _s(stream)))


def select_topk(score, cand_pos, cand_len, k, sel_pos, sel_len, ws=None, stream=None):
    B, P = score.shape
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("csa2_select_topk",
           lib().csa2_select_topk(_p(score), _p(cand_pos), _p(cand_len), B, P, k, _p(sel_pos),
                                  _p(sel_len), _p(ws), nbytes, _s(stream)))


def stream_read(src, sink, stream=None):
    """Read the bytes of tensor `src` once (measurement helper; see
    include/csa2_measure.h)."""
    nbytes = src.numel() * src.element_size()
    _check("csa2_stream_read",
           lib().csa2_stream_read(_p(src), nbytes, _p(sink), sink.numel(), _s(stream)))


def stream_read_sink_words(nbytes: int) -> int:
    return int(lib().csa2_stream_read_sink_words(nbytes))


def empty_kernel(stream=None):
    _check("csa2_empty_kernel", lib().csa2_empty_kernel(_s(stream)))


def handoff_scratch_bytes(groups: int, splits: int) -> int:
    return int(lib().csa2_handoff_scratch_bytes(groups, splits))


def handoff(mode: int, groups: int, splits: int, value: float, scratch, out, stream=None):
    """Measurement helper (include/csa2_measure.h): split partials handed to a
    merge in a second kernel (mode 0) or in the same kernel (modes 1, 2)."""
    nbytes = scratch.numel() * scratch.element_size()
    _check("csa2_handoff", lib().csa2_handoff(mode, groups, splits, float(value), _p(scratch),
                                              nbytes, _p(out), _s(stream)))


def sparse_attn_decode(q, kv_fp4, kv_scale, row_off, lens, max_len, sel_pos, sel_len, k, window,
                       sm_scale, out, lse, ws, stream=None):
    B, Hq, D = q.shape
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("csa2_sparse_attn_decode",
           lib().csa2_sparse_attn_decode(_p(q), _p(kv_fp4), _p(kv_scale), _p(row_off), _p(lens),
                                         int(max_len), _p(sel_pos), _p(sel_len), B, Hq, D, k,
                                         window, float(sm_scale), _p(out), _p(lse), _p(ws),
                                         nbytes, _s(stream)))


ATTN_STATIC_SCRATCH_BYTES = 32 << 20


def sparse_attn_decode_static(q, kv_fp4, kv_scale, row_off, lens, max_len, sel_pos, sel_len, k,
                              window, sm_scale, out, lse, stream=None):
    """csa2_sparse_attn_decode_static: no workspace argument (the library's
    per-GPU static scratch holds the split partials)."""
    B, Hq, D = q.shape
    _check("csa2_sparse_attn_decode_static",
           lib().csa2_sparse_attn_decode_static(_p(q), _p(kv_fp4), _p(kv_scale), _p(row_off),
                                                _p(lens), int(max_len), _p(sel_pos),
                                                _p(sel_len), B, Hq, D, k, window,
                                                float(sm_scale), _p(out), _p(lse), _s(stream)))


# ---- verify blocks: T tokens per sequence (per-token or shared selection) ----

def block_workspace_bytes(op: int, B: int, T: int, shared: bool, max_len: int = 0,
                          total_len: int = 0, H: int = 0, P: int = 0, k: int = 0, Hq: int = 0,
                          D: int = 0, window: int = 0) -> int:
    return int(lib().csa2_block_workspace_bytes(op, B, T, int(shared), max_len, total_len, H, P,
                                                k, Hq, D, window))


def index_full_block(q, w, keys, row_off, lens, max_len, total_len, window, P, shared, pool_pos,
                     pool_score, pool_len, ws, stream=None, k=0, sel_pos=None, sel_len=None):
    """q [B][T][H][Dk]; w [B][T][H]."""
    B, T, H, Dk = q.shape
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("csa2_index_full_block",
           lib().csa2_index_full_block(_p(q), _p(w), _p(keys), _p(row_off), _p(lens), B, T,
                                       int(shared), int(max_len), int(total_len), H, Dk, window,
                                       P, _p(pool_pos), _p(pool_score), _p(pool_len), int(k),
                                       _p(sel_pos), _p(sel_len), _p(ws), nbytes, _s(stream)))


def index_score_block(q, w, keys, row_off, lens, max_len, total_len, window, shared, score, ws,
                      stream=None):
    """q [B][T][H][Dk]; score [B][T][max_len] (per token) or [B][max_len] (shared)."""
    B, T, H, Dk = q.shape
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("csa2_index_score_block",
           lib().csa2_index_score_block(_p(q), _p(w), _p(keys), _p(row_off), _p(lens), B, T,
                                        int(shared), int(max_len), int(total_len), H, Dk, window,
                                        _p(score), _p(ws), nbytes, _s(stream)))


def index_reindex_block(q, w, keys, row_off, cand_pos, cand_len, shared, score, stream=None):
    """q [B][T][H][Dk]; cand_pos / score [lists][P] with lists = B (shared) or B*T."""
    B, T, H, Dk = q.shape
    P = cand_pos.shape[-1]
    _check("csa2_index_reindex_block",
           lib().csa2_index_reindex_block(_p(q), _p(w), _p(keys), _p(row_off), _p(cand_pos),
                                          _p(cand_len), B, T, int(shared), H, Dk, P, _p(score),
                                          _s(stream)))


def sparse_attn_decode_block(q, kv_fp4, kv_scale, row_off, lens, max_len, sel_pos, sel_len, k,
                             window, shared, sm_scale, out, lse, ws, stream=None):
    """q / out [B][T][Hq][D]; sel_pos [B][k] (shared) or [B][T][k]."""
    B, T, Hq, D = q.shape
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("csa2_sparse_attn_decode_block",
           lib().csa2_sparse_attn_decode_block(_p(q), _p(kv_fp4), _p(kv_scale), _p(row_off),
                                               _p(lens), int(max_len), _p(sel_pos), _p(sel_len),
                                               B, T, int(shared), Hq, D, k, window,
                                               float(sm_scale), _p(out), _p(lse), _p(ws), nbytes,
                                               _s(stream)))
