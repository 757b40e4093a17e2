"""Host-side checks of the C-ABI library without a GPU: it loads, exports
every function the header declares, sizes workspaces, and rejects invalid
arguments before launching anything."""
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
    assert {"csa2_kv_append_fp4", "csa2_index_full", "csa2_index_score", "csa2_index_reindex",
            "csa2_select_topk",
            "csa2_sparse_attn_decode", "csa2_workspace_bytes", "csa2_last_error"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_binding_matches_header_parameters(lib):
    """Every declaration's parameter count equals the ctypes binding's."""
    import re
    src = re.sub(r"/\*.*?\*/", "", open(csa2.HEADER).read(), flags=re.S)
    decls = dict(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(([^)]*)\)\s*;", src))
    assert "csa2_index_full" in decls and "csa2_sparse_attn_decode" in decls
    for name, params in decls.items():
        params = params.strip()
        n = 0 if params in ("", "void") else len(params.split(","))
        argtypes = getattr(lib, name).argtypes
        assert argtypes is not None, name
        assert len(argtypes) == n, (name, len(argtypes), n)


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
