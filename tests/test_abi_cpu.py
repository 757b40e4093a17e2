"""Host-side checks of the C-ABI library without a GPU: it loads, exports
every function the header declares, sizes workspaces, and rejects invalid
arguments before launching anything.  Every call here fails validation (the
addresses are fake), so nothing is ever launched, also on a machine with a GPU."""
import ctypes
import os

import pytest

from decode_kv_amd import csa2


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(csa2.LIB_PATH):
        from decode_kv_amd import build
        build.build()
    return csa2.lib()


def test_exports_every_header_function(lib):
    names = csa2.header_functions()
    assert {"csa2_kv_append_fp4", "csa2_append_token", "csa2_index_full", "csa2_index_score",
            "csa2_index_reindex", "csa2_select_topk",
            "csa2_sparse_attn_decode", "csa2_workspace_bytes", "csa2_last_error"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_binding_matches_header_parameters(lib):
    """Every declaration's parameter count equals the ctypes binding's."""
    import re
    decls = dict(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(([^)]*)\)\s*;", csa2.header_source()))
    assert "csa2_index_full" in decls and "csa2_sparse_attn_decode" in decls
    for name, params in decls.items():
        params = params.strip()
        n = 0 if params in ("", "void") else len(params.split(","))
        argtypes = getattr(lib, name).argtypes
        assert argtypes is not None, name
        assert len(argtypes) == n, (name, len(argtypes), n)


def test_stream_read_rejects_bad_arguments(lib):
    f = lib.csa2_stream_read
    assert lib.csa2_stream_read_sink_words(0) == 0
    assert lib.csa2_stream_read_sink_words(1 << 16) == 1
    assert lib.csa2_stream_read_sink_words((1 << 26) + 16) == 1025
    assert f(None, 0, None, 0, None) == csa2.CSA2_OK                   # nothing to read
    assert f(None, 1 << 16, 256, 1, None) == csa2.CSA2_ERR_INVALID
    assert f(264, 1 << 16, 256, 1, None) == csa2.CSA2_ERR_INVALID      # src not 16-aligned
    assert f(256, (1 << 16) + 4, 256, 2, None) == csa2.CSA2_ERR_INVALID
    assert f(256, 1 << 20, 256, 15, None) == csa2.CSA2_ERR_WORKSPACE   # needs 16 words


def test_version_and_error_text(lib):
    assert csa2.version().startswith("csa2-gfx950")
    assert isinstance(csa2.last_error(), str)


def test_workspace_sizes(lib):
    w1 = csa2.workspace_bytes(csa2.OP_INDEX_FULL, 1, 1 << 20, 1 << 20, 64, 16384)
    w2 = csa2.workspace_bytes(csa2.OP_INDEX_FULL, 1, 1 << 21, 1 << 21, 64, 16384)
    assert w1 > 4 * (1 << 20) and w2 > w1 and w1 % 256 == 0
    wk = csa2.workspace_bytes(csa2.OP_INDEX_FULL, 1, 1 << 20, 1 << 20, 64, 16384, 512)
    assert wk > w1 and wk % 256 == 0                 # the selection's own candidate arrays
    assert csa2.workspace_bytes(csa2.OP_INDEX_FULL, 1, 1 << 20, 1 << 20, 64, 16384, 16385) == 0
    assert csa2.workspace_bytes(csa2.OP_SELECT_TOPK, 4, 0, 0, 0, 16384, 512) == 0
    wa1 = csa2.workspace_bytes(csa2.OP_SPARSE_ATTN, 1, 0, 0, 0, 0, 512, 64, 512, 128)
    wa32 = csa2.workspace_bytes(csa2.OP_SPARSE_ATTN, 32, 0, 0, 0, 0, 512, 64, 512, 128)
    assert wa1 > 0 and wa32 > 0
    assert csa2.workspace_bytes(99, 1) == 0 and "unknown op" in csa2.last_error()


V = ctypes.c_void_p


def test_append_rejects_bad_arguments(lib):
    f = lib.csa2_kv_append_fp4
    assert f(None, None, 0, 512, None, None, None) == csa2.CSA2_OK          # n == 0: no-op
    assert f(None, None, 4, 512, None, None, None) == csa2.CSA2_ERR_INVALID
    assert "null" in csa2.last_error()
    assert f(16, 16, 4, 500, 16, 16, None) == csa2.CSA2_ERR_INVALID        # D % 32
    assert f(18, 16, 4, 512, 16, 16, None) == csa2.CSA2_ERR_INVALID        # misaligned
    assert f(16, 16, -1, 512, 16, 16, None) == csa2.CSA2_ERR_INVALID


def test_append_token_rejects_bad_arguments(lib):
    f = lib.csa2_append_token
    #      x    keys_in row_off len  B  nl  layer_rows D   Dk  kv   sc   keys stream
    ok = [256, 256, 256, 256, 2, 20, 1 << 20, 512, 64, 256, 256, 256, None]
    assert f(*ok[:4], 0, *ok[5:]) == csa2.CSA2_OK                       # B == 0: no-op
    for i in (1, 2, 3, 11):                                             # always needed
        bad = list(ok)
        bad[i] = None
        assert f(*bad) == csa2.CSA2_ERR_INVALID and "null" in csa2.last_error(), i
    for i in (0, 9, 10):                                                # needed for layers
        bad = list(ok)
        bad[i] = None
        assert f(*bad) == csa2.CSA2_ERR_INVALID, i
    # no layers: the bf16 rows and the FP4 arrays may be NULL (the call then
    # stops at the next check, Dk, so nothing is launched with these fake addresses)
    bad = list(ok)
    bad[0], bad[9], bad[10], bad[5], bad[8] = None, None, None, 0, 32
    assert f(*bad) == csa2.CSA2_ERR_UNSUPPORTED
    for i, v, code in [(4, -1, csa2.CSA2_ERR_INVALID), (5, -1, csa2.CSA2_ERR_INVALID),
                       (6, -1, csa2.CSA2_ERR_INVALID), (7, 500, csa2.CSA2_ERR_INVALID),
                       (8, 32, csa2.CSA2_ERR_UNSUPPORTED), (4, 70000, csa2.CSA2_ERR_UNSUPPORTED),
                       (0, 264, csa2.CSA2_ERR_INVALID), (1, 264, csa2.CSA2_ERR_INVALID),
                       (11, 264, csa2.CSA2_ERR_INVALID), (9, 258, csa2.CSA2_ERR_INVALID),
                       (2, 260, csa2.CSA2_ERR_INVALID), (3, 258, csa2.CSA2_ERR_INVALID)]:
        bad = list(ok)
        bad[i] = v
        assert f(*bad) == code, (i, v)
        assert "csa2_append_token" in csa2.last_error()


def _full(lib, **kw):
    a = dict(q=256, w=256, keys=256, row_off=256, len=256, B=1, max_len=4096, total_len=4096,
             H=64, Dk=64, window=128, P=1024, pool_pos=256, pool_score=256, pool_len=256,
             k=0, sel_pos=None, sel_len=None, ws=256, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.csa2_index_full(a["q"], a["w"], a["keys"], a["row_off"], a["len"], a["B"],
                               a["max_len"], a["total_len"], a["H"], a["Dk"], a["window"],
                               a["P"], a["pool_pos"], a["pool_score"], a["pool_len"], a["k"],
                               a["sel_pos"], a["sel_len"], a["ws"], a["ws_bytes"], a["stream"])


def test_index_full_rejects_bad_arguments(lib):
    assert _full(lib, B=0) == csa2.CSA2_OK
    assert _full(lib, q=None) == csa2.CSA2_ERR_INVALID
    assert _full(lib, Dk=32) == csa2.CSA2_ERR_UNSUPPORTED
    assert _full(lib, H=0) == csa2.CSA2_ERR_INVALID
    assert _full(lib, H=65) == csa2.CSA2_ERR_INVALID
    assert _full(lib, P=0) == csa2.CSA2_ERR_INVALID
    assert _full(lib, window=-1) == csa2.CSA2_ERR_INVALID
    assert _full(lib, keys=264) == csa2.CSA2_ERR_INVALID
    assert _full(lib, ws=None) == csa2.CSA2_ERR_WORKSPACE
    assert _full(lib, ws_bytes=100) == csa2.CSA2_ERR_WORKSPACE
    assert "workspace" in csa2.last_error()
    assert _full(lib, max_len=1 << 31) == csa2.CSA2_ERR_UNSUPPORTED
    assert _full(lib, k=-1) == csa2.CSA2_ERR_INVALID
    assert _full(lib, k=1025) == csa2.CSA2_ERR_INVALID                      # k > P
    assert _full(lib, k=64) == csa2.CSA2_ERR_INVALID                        # sel_pos NULL
    assert "null" in csa2.last_error()
    assert _full(lib, k=64, sel_pos=256, sel_len=None) == csa2.CSA2_ERR_INVALID


def test_index_score_rejects_bad_arguments(lib):
    f = lib.csa2_index_score
    a = [256, 256, 256, 256, 256, 1, 4096, 4096, 64, 64, 0, 256, 256, 1 << 40, None]
    assert f(*a[:5], 0, *a[6:]) == csa2.CSA2_OK                    # B == 0: no-op
    bad = list(a)
    bad[11] = None                                                  # score
    assert f(*bad) == csa2.CSA2_ERR_INVALID
    bad = list(a)
    bad[9] = 128                                                    # Dk
    assert f(*bad) == csa2.CSA2_ERR_UNSUPPORTED
    bad = list(a)
    bad[10] = -1                                                    # window
    assert f(*bad) == csa2.CSA2_ERR_INVALID
    bad = list(a)
    bad[13] = 64                                                    # ws_bytes
    assert f(*bad) == csa2.CSA2_ERR_WORKSPACE
    assert "csa2_index_score" in csa2.last_error()


def test_reindex_select_attention_reject_bad_arguments(lib):
    r = lib.csa2_index_reindex
    assert r(256, 256, 256, 256, 256, 256, 1, 64, 64, 0, 256, None) == csa2.CSA2_ERR_INVALID
    assert r(256, 256, 256, 256, 256, 256, 1, 64, 16, 16, 256, None) == csa2.CSA2_ERR_UNSUPPORTED
    assert r(None, 256, 256, 256, 256, 256, 1, 64, 64, 16, 256, None) == csa2.CSA2_ERR_INVALID
    s = lib.csa2_select_topk
    assert s(256, 256, 256, 1, 1024, 0, 256, 256, None, 0, None) == csa2.CSA2_ERR_INVALID
    assert s(256, 256, 256, 1, 1024, 2048, 256, 256, None, 0, None) == csa2.CSA2_ERR_INVALID
    assert s(256, 256, 256, 1, 32768, 512, 256, 256, None, 0, None) == csa2.CSA2_ERR_UNSUPPORTED
    a = lib.csa2_sparse_attn_decode
    args = [256, 256, 256, 256, 256, 4096, 256, 256, 1, 64, 512, 512, 128, 0.04, 256, None,
            256, 1 << 40, None]
    bad_d = list(args)
    bad_d[10] = 256
    assert a(*bad_d) == csa2.CSA2_ERR_UNSUPPORTED
    bad_h = list(args)
    bad_h[9] = 24
    assert a(*bad_h) == csa2.CSA2_ERR_INVALID
    no_ws = list(args)
    no_ws[16] = None
    assert a(*no_ws) == csa2.CSA2_ERR_WORKSPACE


def test_attention_rejects_misaligned_cache_and_outputs(lib):
    """The FP4 codes are read in 16-byte pieces and the scale bytes in pairs:
    csa2_sparse_attn_decode rejects a code array that is not 16-byte aligned
    and a scale array that is not 2-byte aligned, before launching anything."""
    a = lib.csa2_sparse_attn_decode
    args = [256, 256, 256, 256, 256, 4096, 256, 256, 1, 64, 512, 512, 128, 0.04, 256, 256,
            256, 1 << 40, None]
    for i, addr in [(1, 264), (1, 260), (1, 257), (2, 257), (0, 264), (14, 264), (3, 260),
                    (4, 258), (6, 258), (7, 258), (15, 258)]:
        bad = list(args)
        bad[i] = addr
        assert a(*bad) == csa2.CSA2_ERR_INVALID, (i, addr)
        assert "misaligned" in csa2.last_error()
    ok = list(args)
    ok[2] = 258                                      # scale bytes: 2-byte alignment suffices
    ok[16] = None                                    # ...so the call gets as far as the workspace
    assert a(*ok) == csa2.CSA2_ERR_WORKSPACE


def test_block_and_session_entries_reject_bad_arguments(lib):
    """Every call below fails its host-side checks, so nothing is launched
    (the pointers are not real device memory)."""
    OK, INV, UNS, WS = csa2.CSA2_OK, csa2.CSA2_ERR_INVALID, csa2.CSA2_ERR_UNSUPPORTED, \
        csa2.CSA2_ERR_WORKSPACE
    p = 1 << 20                                       # 16-aligned stand-in address
    full = lib.csa2_index_full_block
    args = lambda T, shared, B=1, H=64, Dk=64: (p, p, p, p, p, B, T, shared, 100, 100, H, Dk, 128,
                                               64, p, p, p, 0, None, None, p, 1 << 30, None)
    assert full(*args(0, 0)) == INV                  # T < 1
    assert full(*args(5, 2)) == INV                  # shared not 0 / 1
    assert full(*args(1025, 0)) == UNS               # T > 1024
    assert full(*args(5, 0, Dk=32)) == UNS
    assert full(*args(5, 0, B=0)) == OK              # nothing to do
    assert full(*args(1000, 0, B=100)) == UNS        # more than 65535 lists
    assert lib.csa2_index_score_block(p, p, p, p, p, 1, 0, 0, 100, 100, 64, 64, 128, p, p, 1 << 30,
                                      None) == INV
    assert lib.csa2_index_reindex_block(p, p, p, p, p, p, 1, 5, 3, 64, 64, 16, p, None) == INV
    assert lib.csa2_index_reindex_block(p, p, p, p, p, p, 100, 1000, 0, 64, 64, 16, p, None) == UNS
    attn = lib.csa2_sparse_attn_decode_block
    aargs = lambda T, shared, q=p: (q, p, p, p, p, 100, p, p, 1, T, shared, 64, 512, 16, 128,
                                   0.1, p, None, p, 1 << 30, None)
    assert attn(*aargs(0, 0)) == INV and attn(*aargs(2, 5)) == INV
    assert attn(*aargs(1025, 0)) == UNS
    assert attn(*aargs(5, 0, q=p + 8)) == INV        # query rows read in 16-byte pieces
    tok = lib.csa2_append_tokens
    assert tok(p, p, p, p, 1, -1, 3, 100, 512, 64, p, p, p, None) == INV
    assert tok(p, p, p, p, 1, 0, 3, 100, 512, 64, p, p, p, None) == OK   # n == 0
    assert tok(p, p, p, p, 1, 5, 3, 100, 512, 32, p, p, p, None) == UNS   # Dk != 64
    assert tok(p, p, p, p, 1, 5, 3, 100, 500, 64, p, p, p, None) == INV   # D % 32 != 0
    exp = lib.csa2_session_export
    assert exp(p, p, 1, 128, 10, 2, 100, 96, 64, p, p, p, p, p, p, p, None) == UNS   # D % 512
    assert exp(p, p, 1, 128, 10, 2, 100, 512, 64, p + 4, p, p, p, p, p, p, None) == INV
    assert exp(p, p, 1, -1, 10, 2, 100, 512, 64, p, p, p, p, p, p, p, None) == INV
    imp = lib.csa2_session_import
    assert imp(p, p, None, 1, 10, 2, 100, 512, 64, p, p, p, p, p, p, None) == INV
    assert lib.csa2_block_workspace_bytes(csa2.OP_INDEX_FULL, 1, 0, 0, 100, 100, 64, 64, 0, 0, 0,
                                          128) == 0


def test_handoff_rejects_bad_arguments(lib):
    p = 1 << 20
    need = lib.csa2_handoff_scratch_bytes(4, 20)
    assert need == ((4 * 20 * 8192 * 4 + 255) // 256) * 256 + 32
    assert lib.csa2_handoff_scratch_bytes(0, 20) == 0
    h = lib.csa2_handoff
    assert h(3, 4, 20, 1.0, p, need, p, None) == csa2.CSA2_ERR_INVALID
    assert h(0, 4, 20, 1.0, p + 16, need, p, None) == csa2.CSA2_ERR_INVALID   # scratch 256-aligned
    assert h(1, 4, 20, 1.0, p, need - 1, p, None) == csa2.CSA2_ERR_WORKSPACE
    big = lib.csa2_handoff_scratch_bytes(8, 40)
    assert h(1, 8, 40, 1.0, p, big, p, None) == csa2.CSA2_ERR_UNSUPPORTED     # 320 workgroups
